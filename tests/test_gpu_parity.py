"""GPU parity: the HIP path (through the C ABI) against the oracle on the same
seeded bf16 inputs.  Block masks must match bit for bit; outputs and
gradients within max abs 1e-2 and relative L2 5e-3 on valid rows, with padded
rows exactly zero.  Small cases span several tiles and a ragged tail; the
size limits (L = 46080 with a mask, 65536 with key ranges) are checked on
sampled rows.  The benchmark workloads are compared row for row at full size
in test_gpu_full_size.py."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from _gpu import (assert_close, assert_rows, gpu_f64, row_valid, say, to_gpu,
                  to_gpu_bf16)

pytestmark = pytest.mark.gpu

SIGMOID, SOFTMAX, SOFTMAX1 = 0, 1, 2


@pytest.fixture(scope="module")
def va():
    import varlen_attention_amd as va
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    va.load_library()
    return va


def _inputs(seed, B, H, L, d, seq_lens, names=("q", "k", "v")):
    rng = np.random.default_rng(seed)
    return [syn.random_tensor(rng, (B, H, L, d)) for _ in names]


def _bm(va, n_gpu, L, bq, bk, mask_gpu=None, key_range=None):
    """The block matrix, built into a buffer filled with 0xAA first, so an
    entry the builder leaves unwritten shows."""
    shape = (n_gpu.shape[0], -(-L // bq), -(-L // bk))
    out = torch.full(shape, 0xAA, dtype=torch.uint8, device=n_gpu.device)
    va.blockmask_build(n_gpu, L, bq, bk, mask=mask_gpu, key_range=key_range, out=out)
    torch.cuda.synchronize()
    return out


def _handed(q, k, v, n, variant, **kw):
    """What a softmax-family backward is handed by its forward: O rounded to
    bf16 (as the forward stores it) and the LSE in fp32, both from the oracle's
    forward.  The GPU backward and the oracle's backward (o=...) then run on
    the same inputs, so the comparison measures the backward alone; the GPU
    forward is compared on its own.  Returns (O bits, LSE, O on the GPU, LSE
    on the GPU)."""
    o, lse = oracle.fwd(q, k, v, n, variant=variant, **kw)
    o_bits = syn.f32_to_bf16_bits(o.astype(np.float32))
    lse32 = lse.astype(np.float32)
    return o_bits, lse32, to_gpu_bf16(o_bits), to_gpu(lse32, torch.float32)


# --------------------------------------------------------------- block mask
@pytest.mark.parametrize("L,bq,bk", [(128, 32, 32), (100, 64, 32), (1584, 128, 128),
                                     (257, 32, 128), (1, 128, 64)])
def test_blockmask_padding_bitexact(va, L, bq, bk):
    rng = np.random.default_rng(L + bq)
    n = rng.integers(-2, L + 3, size=7).astype(np.int32)
    n[:3] = [0, L, 1]
    say(f"blockmask padding L={L} bq={bq} bk={bk}")
    got = _bm(va, to_gpu(n, torch.int32), L, bq, bk).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.blockmask(n, None, L, bq, bk))


@pytest.mark.parametrize("L,bq,bk,density", [(96, 32, 32, 0.01), (300, 64, 128, 0.002),
                                             (1031, 128, 32, 0.0003), (77, 32, 64, 0.5)])
def test_blockmask_arbitrary_mask_bitexact(va, L, bq, bk, density):
    rng = np.random.default_rng(L)
    B = 4
    n = np.array([L, L // 2, 0, L - 5], np.int32)
    mask = (rng.random((B, L, L)) < density).astype(np.uint8)
    mask[0, L - 1, L - 1] = 1  # corner of the clipped last tile
    say(f"blockmask mask L={L} bq={bq} bk={bk}")
    got = _bm(va, to_gpu(n, torch.int32), L, bq, bk, to_gpu(mask, torch.uint8)).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.blockmask(n, mask, L, bq, bk))


@pytest.mark.parametrize("B,L,bq,bk", [(70, 100, 32, 32), (131, 1100, 128, 64)])
def test_blockmask_mask_many_entries(va, B, L, bq, bk):
    """More than 64 batch entries (the scan finds each workgroup's band over
    several 64-entry steps), lengths from 0 to L: every entry written, the
    units that read and those that only write zeros."""
    rng = np.random.default_rng(B + L)
    n = rng.integers(0, L + 1, size=B).astype(np.int32)
    n[:3] = [0, L, 1]
    mask = (rng.random((B, L, L)) < 0.002).astype(np.uint8)
    say(f"blockmask mask B={B} L={L} bq={bq} bk={bk}")
    got = _bm(va, to_gpu(n, torch.int32), L, bq, bk, to_gpu(mask, torch.uint8)).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.blockmask(n, mask, L, bq, bk))


@pytest.mark.parametrize("L,bk", [(77, 32), (1031, 32), (1031, 128)])
def test_blockmask_mask_end_of_array(va, L, bk):
    """The last row of the whole mask array, its window unaligned (L is not a
    multiple of 16) and its only non-zero bytes in its last 16: the 16-byte
    chunk that would run past the array's end is read byte by byte, and a
    1 KiB window of an unaligned row takes a 65th chunk."""
    B = 3
    n = np.array([L, 5, L], np.int32)
    mask = np.zeros((B, L, L), np.uint8)
    mask[B - 1, L - 1, L - 3] = 1
    mask[B - 1, L - 1, L - 1] = 1
    mask[0, L - 1, min(1023, L - 1)] = 1  # the end of a 1 KiB window in an unaligned row
    say(f"blockmask end of array L={L} bk={bk}")
    got = _bm(va, to_gpu(n, torch.int32), L, 32, bk, to_gpu(mask, torch.uint8)).cpu().numpy()
    want = oracle.blockmask(n, mask, L, 32, bk)
    np.testing.assert_array_equal(got, want)
    assert want[B - 1, -1, -1] & 1 and int((want[B - 1] & 1).sum()) == 1


def test_blockmask_long_documents_full_size(va):
    w = syn.long_packed_docs(tensors=())
    say(f"blockmask {w.name} L={w.L}")
    got = _bm(va, to_gpu(w.seq_lens, torch.int32), w.L, 128, 128,
              to_gpu(w.mask, torch.uint8)).cpu().numpy()
    want = oracle.blockmask(w.seq_lens, w.mask, w.L, 128, 128)
    np.testing.assert_array_equal(got, want)
    assert int((want & 1).sum()) == 885  # kept tiles (seed-0 draw)
    assert int((want >> 1).sum()) == 318  # of which full


# --------------------------------------------------------------- forward, small
FWD_CASES = [
    # d, L, block_q, block_k, variant, bias, with_mask
    (64, 300, 128, 128, SIGMOID, 1, False),
    (64, 300, 64, 64, SIGMOID, 2, False),
    (64, 211, 32, 32, SIGMOID, 0, True),
    (128, 300, 128, 128, SIGMOID, 1, False),
    (128, 257, 128, 64, SIGMOID, 1, True),
    (64, 300, 128, 128, SOFTMAX, 0, False),
    (64, 200, 64, 32, SOFTMAX, 1, True),
    (128, 300, 128, 128, SOFTMAX, 0, True),
    (64, 300, 128, 128, SOFTMAX1, 0, False),
    (128, 190, 32, 64, SOFTMAX1, 2, True),
]


@pytest.mark.parametrize("d,L,bq,bk,variant,bias,with_mask", FWD_CASES)
def test_forward_small(va, d, L, bq, bk, variant, bias, with_mask):
    B, H = 4, 2
    n = np.array([L, L - 37, 1, 0], np.int32)
    q, k, v = _inputs(1000 + d + L + variant, B, H, L, d, n)
    rng = np.random.default_rng(7)
    mask = None
    if with_mask:
        mask = (rng.random((B, L, L)) < 0.3).astype(np.uint8)
        mask[0, 5, :] = 0  # a valid query row with no valid key
        mask[1, :, : L // 2] = 0  # whole tiles empty
    say(f"fwd small d={d} L={L} bq={bq} bk={bk} variant={variant} bias={bias} mask={with_mask}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    bm = _bm(va, n_gpu, L, bq, bk, m_gpu) if with_mask else None
    o, lse = va.sigattn_fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), n_gpu,
                            block_mask=bm, mask=m_gpu, bias=bias, variant=variant,
                            block_q=bq, block_k=bk, return_lse=True)
    torch.cuda.synchronize()
    want, want_lse = oracle.fwd(q, k, v, n, mask=mask, bias=bias, variant=variant)
    assert_rows(gpu_f64(o), want, n, "O")
    if variant != SIGMOID:
        got_lse = lse.cpu().numpy().astype(np.float64)
        valid = row_valid(n, B, L)
        for b in range(B):
            for h in range(H):
                g, wl = got_lse[b, h], want_lse[b, h]
                assert np.array_equal(np.isneginf(g), np.isneginf(wl))
                fin = np.isfinite(wl)
                assert np.all(np.abs(g[fin] - wl[fin]) <= 1e-3 * np.maximum(1, np.abs(wl[fin])))
                assert np.all(np.isneginf(g[~valid[b]]))


@pytest.mark.parametrize("variant,d", [(SOFTMAX, 64), (SOFTMAX1, 64), (SOFTMAX, 128)])
def test_softmax_rising_scores(va, variant, d):
    """Scores that rise along the keys, by about five log2 units per 64-key
    step, with a jump of 40 near the end: the online softmax must move its
    reference maximum (and rescale its state) several times per row, and
    skip the rescale on the steps in between.  O and LSE against the oracle."""
    B, H, L = 2, 2, 700
    n = np.array([L, 333], np.int32)
    rng = np.random.default_rng(17 + d + variant)
    scale = 1.0 / np.sqrt(d)
    q = np.ones((B, H, L, d), np.float32) + 0.05 * rng.standard_normal((B, H, L, d), np.float32)
    # s = scale * q.k ~ 0.06 * c (nats), ~5.5 log2 units per 64 keys; key 650 jumps by 40.
    ramp = 0.06 * np.arange(L, dtype=np.float32)
    ramp[650:] += 40.0
    k = (ramp / (scale * d))[None, None, :, None] * np.ones((B, H, L, d), np.float32)
    k = k + 0.05 * rng.standard_normal((B, H, L, d), np.float32)
    v = rng.standard_normal((B, H, L, d), np.float32)
    q, k, v = (syn.f32_to_bf16_bits(t) for t in (q, k, v))
    say(f"softmax rising scores variant={variant} d={d}")
    n_gpu = to_gpu(n, torch.int32)
    o, lse = va.sigattn_fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), n_gpu, bias=0,
                            variant=variant, return_lse=True)
    torch.cuda.synchronize()
    want, want_lse = oracle.fwd(q, k, v, n, bias=0, variant=variant)
    assert_rows(gpu_f64(o), want, n, "O")
    got_lse = lse.cpu().numpy().astype(np.float64)
    valid = np.broadcast_to(row_valid(n, B, L)[:, None, :], (B, H, L))
    assert np.all(np.isneginf(got_lse[~valid]))
    np.testing.assert_allclose(got_lse[valid], want_lse[valid], rtol=1e-3, atol=1e-3)


@pytest.mark.parametrize("L", [1, 2, 31, 33])
@pytest.mark.parametrize("d,bq,bk", [(64, 32, 128), (128, 128, 32)])
def test_tiny_lengths(va, L, d, bq, bk):
    """Padded lengths from 1 to just past one 32-row step: every variant,
    forward and backward, with padding only and with a causal key-range
    mask, lengths L, L // 2 and 0."""
    B, H = 3, 2
    n = np.array([L, L // 2, 0], np.int32)
    q, k, v, do = _inputs(9000 + L + d, B, H, L, d, n, names="qkvd")
    r = np.arange(L)
    kr = np.broadcast_to(np.stack([np.zeros(L, np.int32), r.astype(np.int32)], 1),
                         (B, L, 2)).copy()
    n_gpu = to_gpu(n, torch.int32)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    for form in ("padding", "causal ranges"):
        kr_np = kr if form != "padding" else None
        kr_gpu = None if kr_np is None else to_gpu(kr_np, torch.int32)
        bm = _bm(va, n_gpu, L, bq, bk, key_range=kr_gpu)
        np.testing.assert_array_equal(bm.cpu().numpy(),
                                      oracle.blockmask(n, None, L, bq, bk, key_range=kr_np))
        for variant in (SIGMOID, SOFTMAX, SOFTMAX1):
            say(f"tiny lengths L={L} d={d} bq={bq} bk={bk} {form} variant={variant}")
            bias = 1 if variant == SIGMOID else 0
            kw = dict(block_mask=bm, key_range=kr_gpu, bias=bias, variant=variant, block_q=bq,
                      block_k=bk)
            o = va.sigattn_fwd(*g[:3], n_gpu, **kw)
            ob = None
            if variant != SIGMOID:  # the backward runs on the oracle's O and LSE
                ob, _, o_in, lse_in = _handed(q, k, v, n, variant, bias=bias, key_range=kr_np)
            grads = va.sigattn_bwd(*g, n_gpu, o=o_in if variant else None,
                                   lse=lse_in if variant else None, **kw)
            torch.cuda.synchronize()
            want, _ = oracle.fwd(q, k, v, n, bias=bias, variant=variant, key_range=kr_np)
            assert_rows(gpu_f64(o), want, n, f"O L={L} {form} variant={variant}")
            ref = oracle.bwd(q, k, v, do, n, bias=bias, variant=variant, key_range=kr_np, o=ob)
            for name, got_t, want_t in zip(("dQ", "dK", "dV"), grads, ref):
                assert_rows(gpu_f64(got_t), want_t, n, f"{name} L={L} {form} variant={variant}")


def test_forward_block_mask_optional_for_padding(va):
    """Without a block mask the tiles come from seq_lens; results are identical."""
    B, H, L, d = 3, 2, 400, 64
    n = np.array([400, 129, 7], np.int32)
    q, k, v = (to_gpu_bf16(t) for t in _inputs(5, B, H, L, d, n))
    n_gpu = to_gpu(n, torch.int32)
    bm = _bm(va, n_gpu, L, 128, 128)
    o1 = va.sigattn_fwd(q, k, v, n_gpu, block_mask=bm)
    o2 = va.sigattn_fwd(q, k, v, n_gpu)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_forward_poisoned_padding_and_determinism(va):
    """NaN in every padded row of Q, K, V changes nothing, and two runs agree bitwise."""
    B, H, L, d = 3, 2, 333, 128
    n = np.array([333, 200, 64], np.int32)
    q, k, v = _inputs(11, B, H, L, d, n)
    qp, kp, vp = q.copy(), k.copy(), v.copy()
    for t in (qp, kp, vp):
        for b in range(B):
            t[b, :, n[b]:] = np.uint16(0x7FC0)
    n_gpu = to_gpu(n, torch.int32)
    for variant in (SIGMOID, SOFTMAX, SOFTMAX1):
        say(f"poison variant={variant}")
        a = va.sigattn_fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), n_gpu, variant=variant)
        bq, bk_, bv = to_gpu_bf16(qp), to_gpu_bf16(kp), to_gpu_bf16(vp)
        b1 = va.sigattn_fwd(bq, bk_, bv, n_gpu, variant=variant)
        b2 = va.sigattn_fwd(bq, bk_, bv, n_gpu, variant=variant)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b1.view(torch.int16))
        assert torch.equal(b1.view(torch.int16), b2.view(torch.int16))


def test_forward_strided_views(va):
    """Q, K, V as views of a packed [B, L, 3, H, d] tensor; O written with its own strides."""
    B, H, L, d = 2, 4, 260, 64
    n = np.array([260, 100], np.int32)
    rng = np.random.default_rng(21)
    packed = syn.random_tensor(rng, (B, L, 3, H, d))
    t = to_gpu_bf16(packed)
    q, k, v = (t[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    out_store = torch.zeros(B, L, H, d, dtype=torch.bfloat16, device="cuda")
    o = out_store.permute(0, 2, 1, 3)
    n_gpu = to_gpu(n, torch.int32)
    va.sigattn_fwd(q, k, v, n_gpu, out=o)
    torch.cuda.synchronize()
    qn, kn, vn = (np.ascontiguousarray(packed[:, :, i].transpose(0, 2, 1, 3)) for i in range(3))
    want, _ = oracle.fwd(qn, kn, vn, n)
    assert_rows(gpu_f64(o), want, n, "O (strided)")


@pytest.mark.parametrize("variant", [SIGMOID, SOFTMAX])
def test_backward_strided_views(va, variant):
    """Q, K, V and dO as views of one packed [B, L, 4, H, d] tensor (row stride
    4 H d); O, dQ, dK and dV written into views of a packed [B, L, 4, H, d]
    output with their own strides."""
    B, H, L, d = 2, 3, 230, 64
    n = np.array([230, 101], np.int32)
    rng = np.random.default_rng(22 + variant)
    packed = syn.random_tensor(rng, (B, L, 4, H, d))
    t = to_gpu_bf16(packed)
    q, k, v, do = (t[:, :, i].permute(0, 2, 1, 3) for i in range(4))
    out_store = torch.zeros(B, L, 4, H, d, dtype=torch.bfloat16, device="cuda")
    o, dq, dk, dv = (out_store[:, :, i].permute(0, 2, 1, 3) for i in range(4))
    n_gpu = to_gpu(n, torch.int32)
    bias = 1 if variant == SIGMOID else 0
    say(f"bwd strided views variant={variant}")
    _, lse = va.sigattn_fwd(q, k, v, n_gpu, out=o, bias=bias, variant=variant, return_lse=True)
    torch.cuda.synchronize()
    qn, kn, vn, don = (np.ascontiguousarray(packed[:, :, i].transpose(0, 2, 1, 3)) for i in range(4))
    want, _ = oracle.fwd(qn, kn, vn, n, bias=bias, variant=variant)
    assert_rows(gpu_f64(o), want, n, "O (strided)")
    ob = None
    if variant != SIGMOID:  # the backward runs on the oracle's O (in the strided view) and LSE
        ob, _, o_in, lse_in = _handed(qn, kn, vn, n, variant, bias=bias)
        o.copy_(o_in)
        lse.copy_(lse_in)
    va.sigattn_bwd(q, k, v, do, n_gpu, bias=bias, variant=variant, dq=dq, dk=dk, dv=dv,
                   o=o if variant else None, lse=lse if variant else None)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.bwd(qn, kn, vn, don, n, bias=bias, variant=variant, o=ob)
    for name, got_t, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), (wq, wk, wv)):
        assert_rows(gpu_f64(got_t), ref, n, f"{name} (strided)")


def test_softmax1_equals_softmax_with_zero_key_on_gpu(va):
    """softmax_1 page: a prepended zero key with a zero value adds 1 to each denominator."""
    B, H, L, d = 2, 2, 190, 64
    n = np.array([190, 77], np.int32)
    q, k, v = _inputs(31, B, H, L, d, n)
    z = np.zeros((B, H, 1, d), np.uint16)
    q2, k2, v2 = (np.concatenate([z, t], axis=2) for t in (q, k, v))
    n_gpu = to_gpu(n, torch.int32)
    o1 = va.sigattn_fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), n_gpu, variant=SOFTMAX1,
                        bias=0)
    o2 = va.sigattn_fwd(to_gpu_bf16(q2), to_gpu_bf16(k2), to_gpu_bf16(v2),
                        to_gpu(n + 1, torch.int32), variant=SOFTMAX, bias=0)
    torch.cuda.synchronize()
    a, b = gpu_f64(o1), gpu_f64(o2)
    for bb in range(B):
        assert_close(a[bb, :, : n[bb]], b[bb, :, 1 : n[bb] + 1], "softmax1 vs prepended zero")


def test_unit_values_row_sums(va):
    B, H, L, d = 2, 2, 300, 64
    n = np.array([300, 150], np.int32)
    q, k, _ = _inputs(41, B, H, L, d, n)
    v = syn.f32_to_bf16_bits(np.ones((B, H, L, d), np.float32))
    n_gpu = to_gpu(n, torch.int32)
    o = gpu_f64(va.sigattn_fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), n_gpu,
                               variant=SOFTMAX, bias=0))
    o1 = gpu_f64(va.sigattn_fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), n_gpu,
                                variant=SOFTMAX1, bias=0))
    for b in range(B):
        assert np.abs(o[b, :, : n[b]] - 1).max() <= 2 ** -7
        assert np.all(o1[b, :, : n[b]] > 0) and np.all(o1[b, :, : n[b]] <= 1)


@pytest.mark.parametrize("d,L,bq,bk", [(64, 257, 128, 128), (128, 257, 128, 64),
                                       (64, 211, 32, 32), (128, 300, 64, 128)])
def test_mask_end_of_batch_entry(va, d, L, bq, bk):
    """Mask entries in the last rows and keys of each batch entry, where a
    tile's mask window runs past the end of the L x L mask: the last row sees
    only its last key, so losing that entry would zero the row (bias 0 keeps
    the weight near 1/2).  Forward and backward against the oracle."""
    B, H = 2, 2
    n = np.array([L, L - 1], np.int32)
    q, k, v, do = _inputs(4000 + d + L, B, H, L, d, n, names="qkvd")
    rng = np.random.default_rng(11)
    mask = (rng.random((B, L, L)) < 0.2).astype(np.uint8)
    for b in range(B):
        nb = int(n[b])
        mask[b, nb - 1, :] = 0
        mask[b, nb - 1, nb - 1] = 1
        mask[b, :, nb - 1] = 1  # every query sees the last key
    say(f"mask end d={d} L={L} bq={bq} bk={bk}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = to_gpu(mask, torch.uint8)
    bm = _bm(va, n_gpu, L, bq, bk, m_gpu)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    o = va.sigattn_fwd(*g[:3], n_gpu, block_mask=bm, mask=m_gpu, bias=0, block_q=bq, block_k=bk)
    dq, dk, dv = va.sigattn_bwd(*g, n_gpu, block_mask=bm, mask=m_gpu, bias=0, block_q=bq,
                                block_k=bk)
    torch.cuda.synchronize()
    want, _ = oracle.fwd(q, k, v, n, mask=mask, bias=0)
    assert_rows(gpu_f64(o), want, n, "O")
    wq, wk, wv = oracle.bwd(q, k, v, do, n, mask=mask, bias=0)
    assert_rows(gpu_f64(dq), wq, n, "dQ")
    assert_rows(gpu_f64(dk), wk, n, "dK")
    assert_rows(gpu_f64(dv), wv, n, "dV")


@pytest.mark.parametrize("d,L,bq,bk,variant", [(64, 300, 64, 64, SIGMOID), (128, 330, 128, 128, SIGMOID),
                                                 (64, 257, 128, 64, SOFTMAX), (128, 200, 64, 128, SOFTMAX1)])
def test_causal_mask_full_tiles(va, d, L, bq, bk, variant):
    """A causal mask has full tiles (bit 1 of the block mask) below the
    diagonal: forward and backward against the oracle, and bit-identical to
    the same call with the full bits cleared (every tile then reads its mask)."""
    B, H = 3, 2
    n = np.array([L, L - 29, bq + 3], np.int32)
    q, k, v, do = _inputs(5000 + d + L + variant, B, H, L, d, n, names="qkvd")
    idx = np.arange(L)
    mask = np.broadcast_to((idx[None, :] <= idx[:, None]).astype(np.uint8), (B, L, L)).copy()
    say(f"causal full tiles d={d} L={L} bq={bq} bk={bk} variant={variant}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = to_gpu(mask, torch.uint8)
    bm = _bm(va, n_gpu, L, bq, bk, m_gpu)
    np.testing.assert_array_equal(bm.cpu().numpy(), oracle.blockmask(n, mask, L, bq, bk))
    assert (bm == 3).any()
    bm01 = bm & 1
    bias = 1 if variant == SIGMOID else 0
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    outs = []
    for blk in (bm, bm01):
        o, lse = va.sigattn_fwd(*g[:3], n_gpu, block_mask=blk, mask=m_gpu, bias=bias,
                                variant=variant, block_q=bq, block_k=bk, return_lse=True)
        grads = va.sigattn_bwd(*g, n_gpu, block_mask=blk, mask=m_gpu, bias=bias, variant=variant,
                               block_q=bq, block_k=bk, o=o if variant else None,
                               lse=lse if variant else None)
        outs.append((o,) + tuple(grads))
    torch.cuda.synchronize()
    for a, b_ in zip(*outs):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))
    want, _ = oracle.fwd(q, k, v, n, mask=mask, bias=bias, variant=variant)
    assert_rows(gpu_f64(outs[0][0]), want, n, "O")
    wq, wk, wv = oracle.bwd(q, k, v, do, n, mask=mask, bias=bias, variant=variant)
    for name, got_t, ref in zip(("dQ", "dK", "dV"), outs[0][1:], (wq, wk, wv)):
        assert_rows(gpu_f64(got_t), ref, n, name)


@pytest.mark.parametrize("d,L,bq,bk,variant,with_mask", [
    (64, 300, 32, 32, SIGMOID, False), (64, 280, 64, 128, SOFTMAX, False),
    (128, 260, 32, 64, SIGMOID, True), (64, 230, 128, 32, SOFTMAX1, True),
    (128, 300, 64, 64, SOFTMAX, False)])
def test_caller_block_mask_per_line(va, d, L, bq, bk, variant, with_mask):
    """A caller's own 0/1 block mask drops tiles whose elements are valid.  A
    workgroup of 128 rows (keys in dK/dV) spans several block-mask lines when
    a block is 32 or 64 wide, and each line must drop exactly its own tiles:
    the oracle takes the block mask as an element mask (each element keeps
    its entry's value), ANDed with the element mask when there is one."""
    B, H = 3, 2
    n = np.array([L, L - 37, bq + 5], np.int32)
    q, k, v, do = _inputs(6000 + d + L + variant, B, H, L, d, n, names="qkvd")
    rng = np.random.default_rng(d + L + bq + bk)
    Tq, Tk = -(-L // bq), -(-L // bk)
    blk = (rng.random((B, Tq, Tk)) < 0.55).astype(np.uint8)
    blk[0, 0, :] = 1
    blk[1, :, 0] = 0
    elem = np.ascontiguousarray(blk.repeat(bq, axis=1).repeat(bk, axis=2)[:, :L, :L])
    mask = None
    if with_mask:
        mask = (rng.random((B, L, L)) < 0.7).astype(np.uint8)
        elem = elem & mask
    say(f"caller block mask d={d} L={L} bq={bq} bk={bk} variant={variant} mask={with_mask}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    bias = 1 if variant == SIGMOID else 0
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    bm = to_gpu(blk, torch.uint8)
    o, lse = va.sigattn_fwd(*g[:3], n_gpu, block_mask=bm, mask=m_gpu, bias=bias, variant=variant,
                            block_q=bq, block_k=bk, return_lse=True)
    grads = va.sigattn_bwd(*g, n_gpu, block_mask=bm, mask=m_gpu, bias=bias, variant=variant,
                           block_q=bq, block_k=bk, o=o if variant else None,
                           lse=lse if variant else None)
    torch.cuda.synchronize()
    want, _ = oracle.fwd(q, k, v, n, mask=elem, bias=bias, variant=variant)
    assert_rows(gpu_f64(o), want, n, "O")
    wq, wk, wv = oracle.bwd(q, k, v, do, n, mask=elem, bias=bias, variant=variant)
    for name, got_t, ref in zip(("dQ", "dK", "dV"), grads, (wq, wk, wv)):
        assert_rows(gpu_f64(got_t), ref, n, name)


def _window_ranges(rng, B, L):
    """Sliding windows of random width per row, some reaching past the row,
    some empty (lo > hi), some clipped at 0 or L - 1."""
    r = np.arange(L)
    lo = r[None, :] - rng.integers(0, 80, size=(B, L))
    hi = r[None, :] + rng.integers(-4, 6, size=(B, L))
    kr = np.stack([lo, hi], axis=2).astype(np.int32)
    if L > 3:
        kr[0, 3] = (9, 2)      # empty
    kr[0, L - 1] = (-7, L + 9)  # whole row, clipped both ways
    return kr


@pytest.mark.parametrize("L,bq,bk", [(300, 64, 64), (257, 128, 32), (129, 32, 128), (1, 128, 64)])
def test_blockmask_from_key_ranges_bitexact(va, L, bq, bk):
    rng = np.random.default_rng(L + bk)
    n = np.array([L, max(L - 50, 0), 1, 0], np.int32)
    kr = _window_ranges(rng, 4, L)
    got = _bm(va, to_gpu(n, torch.int32), L, bq, bk, key_range=to_gpu(kr, torch.int32))
    np.testing.assert_array_equal(got.cpu().numpy(),
                                  oracle.blockmask(n, None, L, bq, bk, key_range=kr))


KEY_RANGE_CASES = [
    # d, L, block_q, block_k, variant, bias
    (64, 300, 128, 128, SIGMOID, 1),
    (64, 211, 32, 64, SIGMOID, 0),
    (128, 257, 128, 64, SIGMOID, 2),
    (64, 230, 64, 32, SOFTMAX, 0),
    (128, 190, 64, 128, SOFTMAX1, 1),
]


@pytest.mark.parametrize("d,L,bq,bk,variant,bias", KEY_RANGE_CASES)
def test_key_range_mask(va, d, L, bq, bk, variant, bias):
    """Key ranges against the oracle (forward and backward), and bit-identical
    to the dense-mask path given the mask the ranges stand for."""
    B, H = 4, 2
    n = np.array([L, L - 37, 1, 0], np.int32)
    q, k, v, do = _inputs(6000 + d + L + variant, B, H, L, d, n, names="qkvd")
    kr = _window_ranges(np.random.default_rng(L * 3 + d), B, L)
    dense = oracle.key_range_mask(kr, L)
    say(f"key ranges d={d} L={L} bq={bq} bk={bk} variant={variant} bias={bias}")
    n_gpu = to_gpu(n, torch.int32)
    kr_gpu = to_gpu(kr, torch.int32)
    m_gpu = to_gpu(dense, torch.uint8)
    bm_r = _bm(va, n_gpu, L, bq, bk, key_range=kr_gpu)
    bm_d = _bm(va, n_gpu, L, bq, bk, m_gpu)
    assert torch.equal(bm_r, bm_d)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    ob = o_in = lse_in = None
    if variant != SIGMOID:  # the backward runs on the oracle's O and LSE
        ob, _, o_in, lse_in = _handed(q, k, v, n, variant, bias=bias, key_range=kr)
    res = []
    for form in ({"key_range": kr_gpu}, {"mask": m_gpu}):
        blk = bm_r if "key_range" in form else bm_d
        o = va.sigattn_fwd(*g[:3], n_gpu, block_mask=blk, bias=bias, variant=variant,
                           block_q=bq, block_k=bk, **form)
        grads = va.sigattn_bwd(*g, n_gpu, block_mask=blk, bias=bias, variant=variant,
                               block_q=bq, block_k=bk, o=o_in, lse=lse_in, **form)
        res.append((o,) + tuple(grads))
    torch.cuda.synchronize()
    for a, b_ in zip(*res):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))
    want, _ = oracle.fwd(q, k, v, n, bias=bias, variant=variant, key_range=kr)
    assert_rows(gpu_f64(res[0][0]), want, n, "O")
    wq, wk, wv = oracle.bwd(q, k, v, do, n, bias=bias, variant=variant, key_range=kr, o=ob)
    for name, got_t, ref in zip(("dQ", "dK", "dV"), res[0][1:], (wq, wk, wv)):
        assert_rows(gpu_f64(got_t), ref, n, name)


# --------------------------------------------------------------- forward, workloads
@pytest.mark.parametrize("variant", [SIGMOID, SOFTMAX, SOFTMAX1])
def test_forward_tiny_workloads(va, variant):
    w = syn.tiny_variants(0, variant)
    say(f"fwd tiny variant={variant}")
    n_gpu = to_gpu(w.seq_lens, torch.int32)
    bm = _bm(va, n_gpu, w.L, w.block_q, w.block_k)
    np.testing.assert_array_equal(bm.cpu().numpy(),
                                  oracle.blockmask(w.seq_lens, None, w.L, 32, 32))
    o = va.sigattn_fwd(to_gpu_bf16(w.q), to_gpu_bf16(w.k), to_gpu_bf16(w.v), n_gpu,
                       block_mask=bm, bias=w.bias, variant=variant, block_q=32, block_k=32)
    torch.cuda.synchronize()
    want, _ = oracle.fwd_tiled(w.q, w.k, w.v, w.seq_lens,
                               oracle.blockmask(w.seq_lens, None, w.L, 32, 32), 32, 32,
                               bias=w.bias, variant=variant)
    assert_rows(gpu_f64(o), want, w.seq_lens, f"O tiny variant {variant}")


# --------------------------------------------------------------- backward
BWD_CASES = [
    # d, L, block_q, block_k, bias, with_mask
    (64, 300, 128, 128, 1, False),
    (64, 230, 64, 32, 2, True),
    (64, 150, 32, 64, 0, False),
    (128, 300, 128, 128, 1, False),
    (128, 201, 64, 128, 1, True),
    (128, 190, 32, 32, 2, True),
]


@pytest.mark.parametrize("d,L,bq,bk,bias,with_mask", BWD_CASES)
def test_backward_small(va, d, L, bq, bk, bias, with_mask):
    B, H = 4, 2
    n = np.array([L, L - 41, 1, 0], np.int32)
    q, k, v, do = _inputs(2000 + d + L, B, H, L, d, n, names="qkvd")
    mask = None
    if with_mask:
        rng = np.random.default_rng(3)
        mask = (rng.random((B, L, L)) < 0.4).astype(np.uint8)
        mask[1, : L // 3, :] = 0
    say(f"bwd small d={d} L={L} bq={bq} bk={bk} bias={bias} mask={with_mask}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    bm = _bm(va, n_gpu, L, bq, bk, m_gpu)
    dq, dk, dv = va.sigattn_bwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), to_gpu_bf16(do),
                                n_gpu, block_mask=bm, mask=m_gpu, bias=bias, block_q=bq,
                                block_k=bk)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.bwd(q, k, v, do, n, mask=mask, bias=bias)
    assert_rows(gpu_f64(dq), wq, n, "dQ")
    assert_rows(gpu_f64(dk), wk, n, "dK")
    assert_rows(gpu_f64(dv), wv, n, "dV")


SCALE_CASES = [
    # d, L, block_q, block_k, variant, bias, scale, element mask
    (64, 300, 128, 128, SIGMOID, 1, 0.3, False),
    (128, 257, 64, 64, SIGMOID, 2, 0.3, True),
    (64, 230, 64, 32, SOFTMAX, 0, 0.3, False),
    (128, 300, 128, 128, SOFTMAX, 0, 0.045, True),
    (64, 190, 32, 128, SOFTMAX1, 0, 0.3, False),
]


@pytest.mark.parametrize("d,L,bq,bk,variant,bias,scale,with_mask", SCALE_CASES)
def test_caller_scale(va, d, L, bq, bk, variant, bias, scale, with_mask):
    """A score scale other than 1/sqrt(d), given through the shape's scale
    field: sigmoid folds it into the register operand and the dK/dQ stores,
    the softmax family applies it in fp32; forward, LSE and all gradients
    against the oracle run with the same scale (the softmax-family backward
    on the oracle's O and LSE, as both backwards are handed them)."""
    B, H = 4, 2
    n = np.array([L, L - 37, 1, 0], np.int32)
    q, k, v, do = _inputs(7000 + d + L, B, H, L, d, n, names="qkvd")
    mask = None
    if with_mask:
        rng = np.random.default_rng(L + d)
        mask = (rng.random((B, L, L)) < 0.5).astype(np.uint8)
        mask[0, 3, :] = 0
    say(f"caller scale d={d} L={L} bq={bq} bk={bk} variant={variant} scale={scale}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    bm = _bm(va, n_gpu, L, bq, bk, m_gpu)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    kw = dict(block_mask=bm, mask=m_gpu, bias=bias, variant=variant, scale=scale, block_q=bq,
              block_k=bk)
    o, lse = va.sigattn_fwd(*g[:3], n_gpu, return_lse=True, **kw)
    ob = None
    if variant != SIGMOID:
        ob, _, o_in, lse_in = _handed(q, k, v, n, variant, mask=mask, bias=bias, scale=scale)
    dq, dk, dv = va.sigattn_bwd(*g, n_gpu, o=o_in if variant else None,
                                lse=lse_in if variant else None, **kw)
    torch.cuda.synchronize()
    want_o, want_l = oracle.fwd(q, k, v, n, mask=mask, bias=bias, variant=variant, scale=scale)
    assert_rows(gpu_f64(o), want_o, n, "O")
    if variant != SIGMOID:
        gl = lse.cpu().numpy().astype(np.float64)
        fin = np.isfinite(want_l)
        assert np.array_equal(np.isneginf(gl), np.isneginf(want_l))
        assert np.all(np.abs(gl[fin] - want_l[fin]) <= 1e-3 * np.maximum(1, np.abs(want_l[fin])))
    wq, wk, wv = oracle.bwd(q, k, v, do, n, mask=mask, bias=bias, variant=variant, scale=scale,
                            o=ob)
    for name, got_t, ref in (("dQ", dq, wq), ("dK", dk, wk), ("dV", dv, wv)):
        assert_rows(gpu_f64(got_t), ref, n, name)


@pytest.mark.parametrize("B,H", [(70, 3), (64, 1), (9, 5)])
def test_many_batch_entries_forward_backward(va, B, H):
    """Dispatch order over many (batch entry, head) pairs: more than 64 batch
    entries (natural order), exactly 64 (sorted in one wave), and pair counts
    that do not divide over 8 XCDs; lengths include 0, 1 and L."""
    L, d = 96, 64
    rng = np.random.default_rng(B * 100 + H)
    n = rng.integers(0, L + 1, size=B).astype(np.int32)
    n[0], n[1], n[-1] = 0, L, 1
    q, k, v, do = _inputs(4000 + B + H, B, H, L, d, n, names="qkvd")
    say(f"many batch entries B={B} H={H}")
    n_gpu = to_gpu(n, torch.int32)
    bm = _bm(va, n_gpu, L, 32, 32)
    args = [to_gpu_bf16(t) for t in (q, k, v)]
    o = va.sigattn_fwd(*args, n_gpu, block_mask=bm, block_q=32, block_k=32)
    dq, dk, dv = va.sigattn_bwd(*args, to_gpu_bf16(do), n_gpu, block_mask=bm, block_q=32,
                                block_k=32)
    torch.cuda.synchronize()
    want_o, _ = oracle.fwd(q, k, v, n)
    assert_rows(gpu_f64(o), want_o, n, "O many batch entries")
    wq, wk, wv = oracle.bwd(q, k, v, do, n)
    assert_rows(gpu_f64(dq), wq, n, "dQ many batch entries")
    assert_rows(gpu_f64(dk), wk, n, "dK many batch entries")
    assert_rows(gpu_f64(dv), wv, n, "dV many batch entries")


SOFT_BWD_CASES = [
    # d, L, block_q, block_k, variant, bias, with_mask
    (64, 300, 128, 128, SOFTMAX, 0, False),
    (64, 300, 128, 128, SOFTMAX1, 0, False),
    (64, 230, 64, 32, SOFTMAX1, 1, True),
    (64, 150, 32, 64, SOFTMAX, 2, True),
    (128, 201, 128, 128, SOFTMAX1, 0, False),
    (128, 190, 64, 128, SOFTMAX, 1, True),
    (128, 230, 32, 64, SOFTMAX, 0, False),
]


@pytest.mark.parametrize("d,L,bq,bk,variant,bias,with_mask", SOFT_BWD_CASES)
def test_backward_softmax_variants(va, d, L, bq, bk, variant, bias, with_mask):
    """Softmax-family backward (dS = P (dP - D), D = rowsum(dO O)) handed the
    same O and LSE as the oracle's backward; lengths L, short, 1 and 0, and
    with an element mask rows that see no key at all."""
    B, H = 4, 2
    n = np.array([L, L - 53, 1, 0], np.int32)
    q, k, v, do = _inputs(3000 + d + L + variant, B, H, L, d, n, names="qkvd")
    mask = None
    if with_mask:
        rng = np.random.default_rng(5)
        mask = (rng.random((B, L, L)) < 0.35).astype(np.uint8)
        mask[0, 7, :] = 0  # a valid query row with no valid key
        mask[1, :, : L // 3] = 0  # whole tiles empty
    say(f"softmax-family bwd d={d} L={L} bq={bq} bk={bk} variant={variant} bias={bias} "
        f"mask={with_mask}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    bm = _bm(va, n_gpu, L, bq, bk, m_gpu)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    ob, _, o, lse = _handed(q, k, v, n, variant, mask=mask, bias=bias)
    dq, dk, dv = va.sigattn_bwd(*g, n_gpu, block_mask=bm, mask=m_gpu, bias=bias, variant=variant,
                                block_q=bq, block_k=bk, o=o, lse=lse)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.bwd(q, k, v, do, n, mask=mask, bias=bias, variant=variant, o=ob)
    assert_rows(gpu_f64(dq), wq, n, "dQ")
    assert_rows(gpu_f64(dk), wk, n, "dK")
    assert_rows(gpu_f64(dv), wv, n, "dV")
    # The two halves give the same bits as the one-launch call.
    dk2, dv2 = va.sigattn_bwd_dkdv(*g, n_gpu, block_mask=bm, mask=m_gpu, bias=bias,
                                   variant=variant, block_q=bq, block_k=bk, o=o, lse=lse)
    dq2 = va.sigattn_bwd_dq(*g, n_gpu, block_mask=bm, mask=m_gpu, bias=bias, variant=variant,
                            block_q=bq, block_k=bk, o=o, lse=lse)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("bq,bk", [(128, 128), (64, 64), (128, 32)])
def test_backward_parts_match_fused(va, bq, bk):
    """sigattn_bwd (one launch for dK/dV and dQ when the tile heights agree,
    two otherwise) equals sigattn_bwd_dkdv + sigattn_bwd_dq bit for bit."""
    B, H, L, d = 5, 3, 290, 64
    n = np.array([290, 0, 161, 33, 128], np.int32)
    q, k, v, do = (to_gpu_bf16(t) for t in _inputs(91, B, H, L, d, n, names="qkvd"))
    n_gpu = to_gpu(n, torch.int32)
    bm = _bm(va, n_gpu, L, bq, bk)
    say(f"bwd parts vs fused bq={bq} bk={bk}")
    dq, dk, dv = va.sigattn_bwd(q, k, v, do, n_gpu, block_mask=bm, block_q=bq, block_k=bk)
    dk2, dv2 = va.sigattn_bwd_dkdv(q, k, v, do, n_gpu, block_mask=bm, block_q=bq, block_k=bk)
    dq2 = va.sigattn_bwd_dq(q, k, v, do, n_gpu, block_mask=bm, block_q=bq, block_k=bk)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("bq,bk", [(128, 128), (64, 32)])
def test_every_output_row_written(va, bq, bk):
    """Outputs start as NaN; afterwards valid rows match the oracle and every
    padded row is exactly 0 (LSE -inf), whichever workgroup wrote it: lengths
    0, L, one short sequence with many padded tiles, and odd lengths."""
    B, H, L, d = 5, 2, 700, 64
    n = np.array([0, 700, 9, 333, 129], np.int32)
    q, k, v, do = _inputs(123, B, H, L, d, n, names="qkvd")
    n_gpu = to_gpu(n, torch.int32)
    bm = _bm(va, n_gpu, L, bq, bk)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    nan = lambda: torch.full_like(g[0], float("nan"))
    say(f"outputs fully written bq={bq} bk={bk}")
    for variant in (SIGMOID, SOFTMAX1):
        o = nan()
        lse = torch.full((B, H, L), float("nan"), dtype=torch.float32, device=g[0].device)
        va.sigattn_fwd(*g[:3], n_gpu, block_mask=bm, variant=variant, bias=0, out=o, lse=lse,
                       block_q=bq, block_k=bk)
        torch.cuda.synchronize()
        want, want_lse = oracle.fwd(q, k, v, n, variant=variant, bias=0)
        assert_rows(gpu_f64(o), want, n, f"O variant {variant}")
        if variant != SIGMOID:
            got = lse.cpu().numpy()
            valid = row_valid(n, B, L)
            for b in range(B):
                assert np.all(np.isneginf(got[b][:, ~valid[b]]))
                assert np.all(np.isfinite(got[b][:, valid[b]]))
    dq, dk, dv = nan(), nan(), nan()
    va.sigattn_bwd(*g, n_gpu, block_mask=bm, dq=dq, dk=dk, dv=dv, block_q=bq, block_k=bk)
    torch.cuda.synchronize()
    wq, wk, wv = oracle.bwd(q, k, v, do, n)
    assert_rows(gpu_f64(dq), wq, n, "dQ")
    assert_rows(gpu_f64(dk), wk, n, "dK")
    assert_rows(gpu_f64(dv), wv, n, "dV")


def test_backward_poison_determinism_and_identities(va):
    B, H, L, d = 3, 2, 333, 64
    n = np.array([333, 180, 40], np.int32)
    q, k, v, do = _inputs(77, B, H, L, d, n, names="qkvd")
    poisoned = [t.copy() for t in (q, k, v, do)]
    for t in poisoned:
        for b in range(B):
            t[b, :, n[b]:] = np.uint16(0x7FC0)
    n_gpu = to_gpu(n, torch.int32)
    g1 = va.sigattn_bwd(*(to_gpu_bf16(t) for t in (q, k, v, do)), n_gpu)
    g2 = va.sigattn_bwd(*(to_gpu_bf16(t) for t in poisoned), n_gpu)
    g3 = va.sigattn_bwd(*(to_gpu_bf16(t) for t in poisoned), n_gpu)
    o = va.sigattn_fwd(*(to_gpu_bf16(t) for t in (q, k, v)), n_gpu)
    torch.cuda.synchronize()
    for a, b, c in zip(g1, g2, g3):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(b.view(torch.int16), c.view(torch.int16))
    # <dQ,Q> = <dK,K> and <dV,V> = <dO,O> from the GPU's own results (no oracle).
    qf, kf, vf, dof = (syn.bf16_bits_to_f32(t).astype(np.float64) for t in (q, k, v, do))
    dq, dk, dv = (gpu_f64(t) for t in g1)
    of = gpu_f64(o)
    for b in range(B):
        nb = n[b]
        for h in range(H):
            a1 = (dq[b, h, :nb] * qf[b, h, :nb]).sum()
            a2 = (dk[b, h, :nb] * kf[b, h, :nb]).sum()
            scale = np.abs(dq[b, h, :nb] * qf[b, h, :nb]).sum()
            assert abs(a1 - a2) <= 2e-2 * scale + 1e-6
            e1 = (dv[b, h, :nb] * vf[b, h, :nb]).sum()
            e2 = (dof[b, h, :nb] * of[b, h, :nb]).sum()
            scale = np.abs(dv[b, h, :nb] * vf[b, h, :nb]).sum()
            assert abs(e1 - e2) <= 2e-2 * scale + 1e-6


def _sampled_fwd_bwd(va, q, k, v, do, n, L, b_rows, gpu_kw, oracle_kw, what):
    """Forward and backward through the C ABI, padded rows exactly zero, and
    the oracle on sampled rows: b_rows holds (batch entry, head, query rows,
    starts of 8-key windows for dK and dV)."""
    n_gpu = to_gpu(n, torch.int32)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    soft = gpu_kw.get("variant", SIGMOID) != SIGMOID
    if soft:  # the softmax backward takes the forward's O and LSE
        o, lse = va.sigattn_fwd(*g[:3], n_gpu, return_lse=True, **gpu_kw)
        dq, dk, dv = va.sigattn_bwd(*g, n_gpu, o=o, lse=lse, **gpu_kw)
    else:
        o = va.sigattn_fwd(*g[:3], n_gpu, **gpu_kw)
        dq, dk, dv = va.sigattn_bwd(*g, n_gpu, **gpu_kw)
    torch.cuda.synchronize()
    B, H = q.shape[:2]
    valid = np.broadcast_to(row_valid(n, B, L)[:, None, :], (B, H, L))
    if soft:
        got_lse = lse.cpu().numpy().astype(np.float64)
        assert np.all(np.isneginf(got_lse[~valid])), f"{what}: padded LSE not -inf"
    outs = {}
    for name, t in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
        outs[name] = t
        assert bool((t.view(torch.int16)[torch.from_numpy(~valid).to(t.device)] == 0).all()), \
            f"{what}: padded {name} rows not zero"
    got = {key: [] for key in outs}
    want = {key: [] for key in outs}
    for b, h, rows, starts in b_rows:
        ro, rl = oracle.fwd_rows(q, k, v, n, b, h, rows, **oracle_kw)
        rq, _, _ = oracle.bwd_rows(q, k, v, do, n, b, h, rows, [], **oracle_kw)
        if soft:
            live = [i for i, r in enumerate(rows) if r < int(n[b])]
            np.testing.assert_allclose(got_lse[b, h, [rows[i] for i in live]], rl[live],
                                       rtol=1e-3, atol=1e-3, err_msg=f"{what} LSE")
        for key, ref in (("O", ro), ("dQ", rq)):
            got[key].append(gpu_f64(outs[key][b, h, rows]))
            want[key].append(ref)
        for c0 in starts:
            cols = list(range(c0, min(c0 + 8, L)))
            _, rk, rv = oracle.bwd_rows(q, k, v, do, n, b, h, [], cols, **oracle_kw)
            for key, ref in (("dK", rk), ("dV", rv)):
                got[key].append(gpu_f64(outs[key][b, h, cols]))
                want[key].append(ref)
    for key in got:
        assert_close(np.concatenate(got[key]), np.concatenate(want[key]), f"{what} {key}")


def _band_rows(rng, nb, L, extra=()):
    rows = {0, 1, nb - 1, min(nb, L - 1)} | set(extra)
    rows |= set(rng.integers(0, max(nb, 1), size=6).tolist())
    return sorted(r for r in rows if 0 <= r < L)


def test_max_masked_length(va):
    """The longest padded length accepted with an element mask, with two
    batch entries: the second entry's mask runs past 2^31 bytes from the
    first's.  A causal band of 400 keys (with full tiles) keeps the work
    small; the block mask is compared bit for bit, outputs and gradients on
    sampled rows, including rows past the 2^31-byte mark and fully masked
    rows."""
    L, B, H, d, win = va.MAX_MASKED_L, 2, 1, 64, 400
    n = np.array([L, L - 1001], np.int32)
    rng = np.random.default_rng(46)
    q, k, v, do = (syn.random_tensor(rng, (B, H, L, d)) for _ in range(4))
    mask = np.zeros((B, L, L), np.uint8)
    for r in range(L):
        mask[:, r, max(0, r - win + 1):r + 1] = 1
    mask[1, 30000:30100, :] = 0
    say(f"max masked length L={L}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = to_gpu(mask, torch.uint8)
    bm = _bm(va, n_gpu, L, 128, 128, m_gpu)
    want_bm = oracle.blockmask(n, mask, L, 128, 128)
    assert (want_bm == 3).any()
    np.testing.assert_array_equal(bm.cpu().numpy(), want_bm)
    b_rows = [(0, 0, _band_rows(rng, L, L), (0, 20000, L - 8)),
              (1, 0, _band_rows(rng, int(n[1]), L, extra=(30000, 30099, 40000, L - 1002)),
               (29996, 40000, int(n[1]) - 5))]
    _sampled_fwd_bwd(va, q, k, v, do, n, L, b_rows, dict(block_mask=bm, mask=m_gpu),
                     dict(mask=mask), "max masked length")


def test_key_ranges_past_max_masked_length(va):
    """Key ranges carry no L x L mask, so they go past the dense mask's
    length limit: L = 65536 with sliding windows (some empty, some reaching
    past the row), block mask bit for bit, sampled rows against the oracle
    with the ranges written out as an element mask."""
    L, B, H, d = 65536, 1, 2, 64
    n = np.array([60001], np.int32)
    rng = np.random.default_rng(65)
    q, k, v, do = (syn.random_tensor(rng, (B, H, L, d)) for _ in range(4))
    kr = _window_ranges(rng, B, L)
    kr[0, 50000:50010] = (10, 5)  # empty rows
    say(f"key ranges past max masked length L={L}")
    n_gpu = to_gpu(n, torch.int32)
    kr_gpu = to_gpu(kr, torch.int32)
    bm = _bm(va, n_gpu, L, 128, 128, key_range=kr_gpu)
    elem = oracle.key_range_mask(kr, L)  # what the ranges stand for, written out once
    np.testing.assert_array_equal(bm.cpu().numpy(), oracle.blockmask(n, elem, L, 128, 128))
    b_rows = [(0, h, _band_rows(rng, int(n[0]), L, extra=(50000, 50009, 59999)),
               (0, 49996, int(n[0]) - 4)) for h in range(H)]
    _sampled_fwd_bwd(va, q, k, v, do, n, L, b_rows, dict(block_mask=bm, key_range=kr_gpu),
                     dict(mask=elem), "key ranges L=65536")


def test_long_documents_key_ranges_full_size(va):
    """The causal packed-document mask as key ranges (8 bytes per row instead
    of an L x L mask) at B8 H16 d128: the same block mask and bit-identical
    forward and backward results as the dense mask."""
    w = syn.long_packed_docs(0, tensors=("q", "k", "v", "do"))
    say(f"key ranges full {w.name} L={w.L}")
    n_gpu = to_gpu(w.seq_lens, torch.int32)
    kr_gpu = to_gpu(w.key_range, torch.int32)
    m_gpu = to_gpu(w.mask, torch.uint8)
    bm_r = _bm(va, n_gpu, w.L, 128, 128, key_range=kr_gpu)
    bm_d = _bm(va, n_gpu, w.L, 128, 128, m_gpu)
    assert torch.equal(bm_r, bm_d)
    g = [to_gpu_bf16(t) for t in (w.q, w.k, w.v, w.do)]
    res = []
    for form, blk in (({"key_range": kr_gpu}, bm_r), ({"mask": m_gpu}, bm_d)):
        o = va.sigattn_fwd(*g[:3], n_gpu, block_mask=blk, **form)
        res.append((o,) + tuple(va.sigattn_bwd(*g, n_gpu, block_mask=blk, **form)))
    torch.cuda.synchronize()
    for a, b_ in zip(*res):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))


# --------------------------------------------------------------- differential attention
DIFF_CASES = [
    # d, L, block_q, block_k, mask form ("none", "dense", "range"), lambda
    (64, 300, 128, 128, "none", 0.8),
    (64, 211, 64, 32, "dense", 0.37),
    (128, 257, 128, 64, "range", 0.6),
    (128, 190, 32, 128, "dense", -0.25),
    (64, 150, 32, 64, "range", 1.0),
    (128, 333, 128, 128, "none", 0.8),
]


@pytest.mark.parametrize("d,L,bq,bk,form,lam", DIFF_CASES)
def test_diff_forward(va, d, L, bq, bk, form, lam):
    """Differential attention against the oracle (O and both LSEs); with
    lambda = 0 the output and LSEs match two softmax calls to rounding."""
    B, H = 4, 2
    n = np.array([L, L - 37, 1, 0], np.int32)
    q1, k1, q2, k2, v = _inputs(7000 + d + L, B, H, L, d, n, names="abcde")
    rng = np.random.default_rng(L + d)
    mask = kr = None
    if form == "dense":
        mask = (rng.random((B, L, L)) < 0.4).astype(np.uint8)
        mask[0, 5, :] = 0
    elif form == "range":
        kr = _window_ranges(rng, B, L)
    say(f"diff fwd d={d} L={L} bq={bq} bk={bk} form={form} lam={lam}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    kr_gpu = None if kr is None else to_gpu(kr, torch.int32)
    bm = _bm(va, n_gpu, L, bq, bk, m_gpu, key_range=kr_gpu)
    g = [to_gpu_bf16(t) for t in (q1, k1, q2, k2, v)]
    kw = dict(block_mask=bm, mask=m_gpu, key_range=kr_gpu, block_q=bq, block_k=bk)
    o, l1, l2 = va.sigattn_diff_fwd(*g, n_gpu, lam, return_lse=True, **kw)
    o0, z1, z2 = va.sigattn_diff_fwd(*g, n_gpu, 0.0, return_lse=True, **kw)
    s1, t1 = va.sigattn_fwd(g[0], g[1], g[4], n_gpu, variant=SOFTMAX, bias=0, return_lse=True, **kw)
    _, t2 = va.sigattn_fwd(g[2], g[3], g[4], n_gpu, variant=SOFTMAX, bias=0, return_lse=True, **kw)
    torch.cuda.synchronize()
    # lambda = 0 is map 1's softmax.  Not bit for bit: the one-map loop moves
    # its reference maximum lazily and the two-map loop every tile (and at
    # d = 128 the two-map loop steps 32 keys at a time), so weights round
    # differently; the log-sum-exps agree to fp32 rounding.
    assert_rows(gpu_f64(o0), gpu_f64(s1), n, "O (lambda 0) vs softmax")
    for got_l, ref_l in ((z1, t1), (z2, t2)):
        gl, rl = got_l.cpu().numpy(), ref_l.cpu().numpy()
        assert np.array_equal(np.isneginf(gl), np.isneginf(rl))
        fin = np.isfinite(rl)
        np.testing.assert_allclose(gl[fin], rl[fin], rtol=1e-5, atol=1e-5)
    want, w1, w2 = oracle.diff_fwd(q1, k1, q2, k2, v, n, lam, mask=mask, key_range=kr)
    assert_rows(gpu_f64(o), want, n, "O")
    valid = row_valid(n, B, L)
    for got_l, want_l in ((l1, w1), (l2, w2)):
        gl = got_l.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(gl), np.isneginf(want_l))
        fin = np.isfinite(want_l)
        assert np.all(np.abs(gl[fin] - want_l[fin]) <= 1e-3 * np.maximum(1, np.abs(want_l[fin])))
        assert np.all(np.isneginf(gl[~np.broadcast_to(valid[:, None, :], gl.shape)]))


DIFF_BWD_CASES = [
    # d, L, block_q, block_k, mask form, lambda (d = 64: both maps in one pass,
    # in one launch when block_q == block_k)
    (64, 300, 128, 128, "none", 0.8),
    (64, 230, 64, 32, "dense", 0.37),
    (64, 257, 128, 128, "range", 0.5),
    (64, 190, 64, 64, "dense", -0.4),
    (128, 201, 128, 128, "range", 0.6),
    (128, 190, 64, 128, "dense", -0.3),
    (128, 333, 128, 128, "none", 0.8),
]


@pytest.mark.parametrize("d,L,bq,bk,form,lam", DIFF_BWD_CASES)
def test_diff_backward(va, d, L, bq, bk, form, lam):
    """Differential attention backward against the oracle, both handed the same
    per-map outputs and LSEs (each map's forward output is compared first);
    map 1's gradients equal sigattn_bwd's softmax backward bit for bit."""
    B, H = 4, 2
    n = np.array([L, L - 53, 1, 0], np.int32)
    q1, k1, q2, k2, v, do = _inputs(8000 + d + L, B, H, L, d, n, names="abcdef")
    rng = np.random.default_rng(L * 7 + d)
    mask = kr = None
    if form == "dense":
        mask = (rng.random((B, L, L)) < 0.4).astype(np.uint8)
        mask[0, 5, :] = 0
    elif form == "range":
        kr = _window_ranges(rng, B, L)
    say(f"diff bwd d={d} L={L} bq={bq} bk={bk} form={form} lam={lam}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    kr_gpu = None if kr is None else to_gpu(kr, torch.int32)
    bm = _bm(va, n_gpu, L, bq, bk, m_gpu, key_range=kr_gpu)
    g = [to_gpu_bf16(t) for t in (q1, k1, q2, k2, v, do)]
    kw = dict(block_mask=bm, mask=m_gpu, key_range=kr_gpu, block_q=bq, block_k=bk)
    o, l1, l2, o1, o2 = va.sigattn_diff_fwd(*g[:5], n_gpu, lam, return_maps=True, **kw)
    w1, _ = oracle.fwd(q1, k1, v, n, mask=mask, key_range=kr, bias=0, variant=SOFTMAX)
    torch.cuda.synchronize()
    assert_rows(gpu_f64(o1), w1, n, "O1")
    # The backward runs on the oracle's per-map outputs and LSEs.
    ob1, _, o1, l1 = _handed(q1, k1, v, n, SOFTMAX, mask=mask, key_range=kr, bias=0)
    ob2, _, o2, l2 = _handed(q2, k2, v, n, SOFTMAX, mask=mask, key_range=kr, bias=0)
    grads = va.sigattn_diff_bwd(*g, o1, o2, l1, l2, n_gpu, lam, **kw)
    ref1 = va.sigattn_bwd(g[0], g[1], g[4], g[5], n_gpu, variant=SOFTMAX, bias=0, o=o1, lse=l1,
                          **kw)
    torch.cuda.synchronize()
    assert torch.equal(grads[0].view(torch.int16), ref1[0].view(torch.int16))
    assert torch.equal(grads[1].view(torch.int16), ref1[1].view(torch.int16))
    want = oracle.diff_bwd(q1, k1, q2, k2, v, do, n, lam, mask=mask, key_range=kr, o1=ob1, o2=ob2)
    for name, got_t, ref in zip(("dQ1", "dK1", "dQ2", "dK2", "dV"), grads, want):
        assert_rows(gpu_f64(got_t), ref, n, name)


@pytest.mark.parametrize("d,bq", [(64, 128), (64, 64), (128, 128)])
def test_diff_backward_caller_scale(va, d, bq):
    """Differential attention with a score scale other than 1/sqrt(d) (0.3):
    forward and all five gradients against the oracle with the same scale.
    d = 64 runs both maps in one pass (the scale and -lambda enter at the
    dK2 and dQ2 stores), d = 128 as two softmax backward launches."""
    B, H, L, lam, scale = 3, 2, 260, 0.6, 0.3
    n = np.array([L, 131, 0], np.int32)
    q1, k1, q2, k2, v, do = _inputs(6100 + d + bq, B, H, L, d, n, names="abcdef")
    say(f"diff bwd caller scale d={d} bq={bq} scale={scale}")
    n_gpu = to_gpu(n, torch.int32)
    bm = _bm(va, n_gpu, L, bq, bq)
    g = [to_gpu_bf16(t) for t in (q1, k1, q2, k2, v, do)]
    kw = dict(block_mask=bm, block_q=bq, block_k=bq, scale=scale)
    o = va.sigattn_diff_fwd(*g[:5], n_gpu, lam, **kw)
    want_o, _, _ = oracle.diff_fwd(q1, k1, q2, k2, v, n, lam, scale=scale)
    torch.cuda.synchronize()
    assert_rows(gpu_f64(o), want_o, n, "O")
    ob1, _, o1, l1 = _handed(q1, k1, v, n, SOFTMAX, bias=0, scale=scale)
    ob2, _, o2, l2 = _handed(q2, k2, v, n, SOFTMAX, bias=0, scale=scale)
    grads = va.sigattn_diff_bwd(*g, o1, o2, l1, l2, n_gpu, lam, **kw)
    torch.cuda.synchronize()
    want = oracle.diff_bwd(q1, k1, q2, k2, v, do, n, lam, scale=scale, o1=ob1, o2=ob2)
    for name, got_t, ref in zip(("dQ1", "dK1", "dQ2", "dK2", "dV"), grads, want):
        assert_rows(gpu_f64(got_t), ref, n, name)


@pytest.mark.parametrize("variant", [SIGMOID, SOFTMAX])
def test_hip_graph_capture_and_replay(va, variant):
    """The whole step (block mask and schedule, forward, backward) captured in
    one HIP graph through torch: the library allocates nothing and records no memset,
    so replays (with eager work and synchronisations between them) give the
    eager results bit for bit."""
    B, H, L, d = 4, 2, 300, 64
    n = np.array([300, 177, 31, 0], np.int32)
    q, k, v, do = _inputs(4242 + variant, B, H, L, d, n, names="qkvd")
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    n_gpu = to_gpu(n, torch.int32)
    bias = 1 if variant == SIGMOID else 0
    say(f"graph capture variant={variant}")

    def step(out):
        bm, sched = va.blockmask_build(n_gpu, L, 64, 64, out=out["bm"], heads=H,
                                       schedule=out["sched"])
        va.sigattn_fwd(*g[:3], n_gpu, block_mask=bm, schedule=sched, bias=bias, variant=variant,
                       block_q=64, block_k=64, out=out["o"], lse=out["lse"])
        va.sigattn_bwd(*g, n_gpu, block_mask=bm, schedule=sched, bias=bias, variant=variant,
                       block_q=64, block_k=64, dq=out["dq"], dk=out["dk"], dv=out["dv"],
                       o=out["o"] if variant else None, lse=out["lse"] if variant else None)

    def buffers():
        t = {key: torch.empty_like(g[0]) for key in ("o", "dq", "dk", "dv")}
        t["lse"] = torch.empty((B, H, L), dtype=torch.float32, device=g[0].device)
        t["bm"] = torch.empty((B, -(-L // 64), -(-L // 64)), dtype=torch.uint8,
                              device=g[0].device)
        t["sched"] = torch.empty(va.schedule_bytes(B, H, L, 64, 64), dtype=torch.uint8,
                                 device=g[0].device)
        return t

    eager = buffers()
    step(eager)
    torch.cuda.synchronize()
    cap = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture, as torch asks
        step(cap)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cap)
    for rep in range(3):
        for t in cap.values():
            t.zero_()
        junk = buffers()
        step(junk)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key in ("bm", "sched", "o", "dq", "dk", "dv"):
            assert torch.equal(cap[key].view(torch.uint8), eager[key].view(torch.uint8)), \
                f"replay {rep}: {key} differs from the eager run"
        if variant:
            assert torch.equal(cap["lse"], eager["lse"]), f"replay {rep}: lse differs"


def test_two_streams_at_once(va):
    """The library keeps no state between calls: two problems launched on two
    streams, interleaved, give what each gives alone, bit for bit."""
    B, H, d = 3, 2, 64
    cases = []
    for seed, L in ((1, 257), (2, 400)):
        n = np.array([L, L // 3, 7], np.int32)
        q, k, v, do = _inputs(4300 + seed, B, H, L, d, n, names="qkvd")
        cases.append(([to_gpu_bf16(t) for t in (q, k, v, do)], to_gpu(n, torch.int32), L))
    say("two streams")

    def run(case, stream):
        g, n_gpu, L = case
        with torch.cuda.stream(stream):
            bm = va.blockmask_build(n_gpu, L, 128, 128)
            o = va.sigattn_fwd(*g[:3], n_gpu, block_mask=bm)
            grads = va.sigattn_bwd(*g, n_gpu, block_mask=bm)
        return (o,) + tuple(grads)

    alone = [run(c, torch.cuda.current_stream()) for c in cases]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        together = [run(cases[0], s1), run(cases[1], s2)]
        torch.cuda.synchronize()
        for a, b_ in zip(alone, together):
            for x, y in zip(a, b_):
                assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_binding_rejects_malformed_tensors(va):
    """The binding checks dtypes, shapes, strides and the softmax backward's
    extra inputs before anything reaches the library; each case raises and
    launches nothing."""
    dev = torch.device("cuda:0")
    B, H, L, d = 2, 2, 64, 64
    q = torch.zeros(B, H, L, d, dtype=torch.bfloat16, device=dev)
    n = torch.full((B,), L, dtype=torch.int32, device=dev)
    say("binding argument checks")
    with pytest.raises(TypeError):
        va.sigattn_fwd(q.float(), q, q, n)                       # dtype
    with pytest.raises(ValueError):
        va.sigattn_fwd(q, q[:, :, :32], q, n)                    # shape
    with pytest.raises(ValueError):
        va.sigattn_fwd(q, q.transpose(2, 3).contiguous().transpose(2, 3), q, n)  # d stride
    with pytest.raises(ValueError):
        va.sigattn_fwd(q, q, q, n, mask=torch.zeros(B, L, L - 1, dtype=torch.uint8, device=dev),
                       block_mask=va.blockmask_build(n, L))       # mask shape
    with pytest.raises(ValueError):
        va.sigattn_fwd(q, q, q, n, block_mask=torch.zeros(B, 3, 3, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        va.sigattn_bwd(q, q, q, q, n, variant=SOFTMAX)           # softmax needs o and lse
    with pytest.raises(ValueError):
        va.sigattn_fwd(q, q, q, n, lse=torch.zeros(B, H, L + 1, device=dev), variant=SOFTMAX)
    with pytest.raises(ValueError):
        va.blockmask_build(n, L, key_range=torch.zeros(B, L, 3, dtype=torch.int32, device=dev))
    # seq_lens must hold exactly B lengths: the kernels read seq_lens[0 .. B-1].
    short, wide = n[:1], n.view(1, B)
    with pytest.raises(ValueError):
        va.sigattn_fwd(q, q, q, short)
    with pytest.raises(ValueError):
        va.sigattn_fwd(q, q, q, wide)
    with pytest.raises(ValueError):
        va.sigattn_bwd(q, q, q, q, short)
    with pytest.raises(ValueError):
        va.sigattn_bwd_dkdv(q, q, q, q, short)
    with pytest.raises(ValueError):
        va.sigattn_bwd_dq(q, q, q, q, torch.cat([n, n]))
    with pytest.raises(ValueError):
        va.sigattn_diff_fwd(q, q, q, q, q, short, 0.5)
    with pytest.raises(ValueError):
        va.sigattn_diff_bwd(q, q, q, q, q, q, q, q, torch.zeros(B, H, L, device=dev),
                            torch.zeros(B, H, L, device=dev), short, 0.5)
    with pytest.raises(ValueError):
        va.blockmask_build(wide, L)


@pytest.mark.parametrize("variant", [SIGMOID, SOFTMAX1])
def test_lengths_outside_zero_to_L_are_clamped(va, variant):
    """seq_lens is device memory and not checked on the host: a negative
    length acts as 0 and one past L as L, in the block mask, the forward and
    the backward alike."""
    B, H, L, d = 4, 2, 150, 64
    n = np.array([-5, L + 7, L, 3], np.int32)
    q, k, v, do = _inputs(4400 + variant, B, H, L, d, np.clip(n, 0, L), names="qkvd")
    say(f"clamped lengths variant={variant}")
    n_gpu = to_gpu(n, torch.int32)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    bm = _bm(va, n_gpu, L, 64, 64)
    np.testing.assert_array_equal(bm.cpu().numpy(), oracle.blockmask(n, None, L, 64, 64))
    bias = 1 if variant == SIGMOID else 0
    kw = dict(block_mask=bm, bias=bias, variant=variant, block_q=64, block_k=64)
    o, lse = va.sigattn_fwd(*g[:3], n_gpu, return_lse=True, **kw)
    grads = va.sigattn_bwd(*g, n_gpu, o=o if variant else None, lse=lse if variant else None, **kw)
    torch.cuda.synchronize()
    nc = np.clip(n, 0, L).astype(np.int32)
    want, _ = oracle.fwd(q, k, v, n, bias=bias, variant=variant)
    assert_rows(gpu_f64(o), want, nc, "O")
    for name, got_t, ref in zip(("dQ", "dK", "dV"), grads,
                                oracle.bwd(q, k, v, do, n, bias=bias, variant=variant)):
        assert_rows(gpu_f64(got_t), ref, nc, name)
