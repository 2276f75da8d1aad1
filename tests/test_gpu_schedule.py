"""The work schedule blockmask_build writes beside the block mask (work items
per XCD, longest sequence first, and zero items for the fully padded tiles;
kept-entry lists per 128-row group): bit for bit the oracle's schedule, and
attention results bit for bit those without it (forward, backward in one
launch and in two, every variant, every mask form and block size,
differential attention), every padded row written."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from _gpu import decode_schedule, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

SIGMOID, SOFTMAX, SOFTMAX1 = 0, 1, 2


@pytest.fixture(scope="module")
def va():
    import varlen_attention_amd as va
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    va.load_library()
    return va


def _window_ranges(rng, B, L):
    kr = np.zeros((B, L, 2), np.int32)
    for b in range(B):
        lo = np.maximum(np.arange(L) - rng.integers(0, 300, L), 0)
        kr[b, :, 0], kr[b, :, 1] = lo, np.arange(L) + rng.integers(-5, 40, L)
    return kr


def _check_packed_mask(buf, mask, n, B, H, L, bq, bk):
    """The mask packed to bits at the end of the schedule (after the lists,
    at a 16-byte boundary): bit t of word w of row r is entry (r, 32 w + t).
    Compared with the mask for rows and keys below n (the rest is
    unspecified)."""
    G = -(-L // 128)
    Tq, Tk = -(-L // bq), -(-L // bk)
    slots1 = 8 * (-(-(B * H) // 8)) * G
    off = -(-(16 * 3 * slots1 + 4 * B * G * (Tk + 1 + Tq + 1)) // 16) * 16
    W = -(-L // 32)
    words = np.frombuffer(buf[off:off + 4 * B * L * W].tobytes(), dtype=np.uint32)
    words = words.reshape(B, L, W)
    for b in range(B):
        nb = int(np.clip(n[b], 0, L))
        if nb == 0:
            continue
        got = np.unpackbits(words[b, :nb].view(np.uint8), axis=1, bitorder="little")[:, :nb]
        np.testing.assert_array_equal(got, (mask[b, :nb, :nb] != 0).astype(np.uint8))


SCHED_CASES = [
    # B, H, L, block_q, block_k, mask form
    (32, 8, 1584, 128, 128, "none"),   # the single-cell shapes
    (5, 3, 700, 32, 128, "dense"),
    (7, 11, 333, 64, 32, "range"),
    (70, 2, 260, 128, 64, "none"),     # more than 64 batch entries
    (3, 1, 1, 32, 32, "none"),
    (9, 5, 1030, 128, 128, "dense"),
]


@pytest.mark.parametrize("B,H,L,bq,bk,form", SCHED_CASES)
def test_schedule_matches_oracle(va, B, H, L, bq, bk, form):
    rng = np.random.default_rng(B * 1000 + L)
    if (B, H, L) == (32, 8, 1584):
        n = syn.single_cell(0, tensors=()).seq_lens
    else:
        n = rng.integers(-3, L + 3, size=B).astype(np.int32)
        n[0], n[-1] = L, 0
    mask = kr = None
    if form == "dense":
        mask = (rng.random((B, L, L)) < 0.003).astype(np.uint8)
        mask[0, : L // 2, : L // 2] = 1
    elif form == "range":
        kr = _window_ranges(rng, B, L)
    say(f"schedule B={B} H={H} L={L} bq={bq} bk={bk} form={form}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    kr_gpu = None if kr is None else to_gpu(kr, torch.int32)
    bm, sched = va.blockmask_build(n_gpu, L, bq, bk, mask=m_gpu, key_range=kr_gpu, heads=H)
    torch.cuda.synchronize()
    assert sched.numel() == va.schedule_bytes(B, H, L, bq, bk, dense_mask=mask is not None)
    if mask is not None:
        _check_packed_mask(sched.cpu().numpy(), mask, n, B, H, L, bq, bk)
    want_bm = oracle.blockmask(n, mask, L, bq, bk, key_range=kr)
    np.testing.assert_array_equal(bm.cpu().numpy(), want_bm)
    got = decode_schedule(sched.cpu().numpy(), B, H, L, bq, bk)
    want = oracle.schedule(n, want_bm, H, L, bq, bk)
    for key in ("items1", "items2", "qlists", "klists"):
        assert got[key] == want[key], key


OUT_CASES = [
    # d, L, block_q, block_k, variant, bias, mask form
    (64, 300, 128, 128, SIGMOID, 1, "none"),
    (64, 257, 64, 64, SOFTMAX, 0, "none"),
    (128, 300, 32, 128, SIGMOID, 2, "dense"),
    (64, 290, 128, 32, SOFTMAX1, 0, "range"),
    (128, 190, 64, 64, SOFTMAX, 1, "range"),
    (64, 400, 32, 32, SIGMOID, 1, "dense"),
    (64, 333, 64, 64, SOFTMAX, 0, "dense"),     # rows not 16-byte aligned
    (128, 333, 128, 128, SOFTMAX1, 0, "dense"),
]


@pytest.mark.parametrize("d,L,bq,bk,variant,bias,form", OUT_CASES)
def test_outputs_identical_with_schedule(va, d, L, bq, bk, variant, bias, form):
    B, H = 6, 3
    n = np.array([L, L - 41, 1, 0, L // 2, 129], np.int32)
    rng = np.random.default_rng(d + L + bq)
    q, k, v, do = (syn.random_tensor(rng, (B, H, L, d)) for _ in range(4))
    mask = kr = None
    if form == "dense":
        mask = (rng.random((B, L, L)) < 0.4).astype(np.uint8)
        mask[1, :, : L // 2] = 0
    elif form == "range":
        kr = _window_ranges(rng, B, L)
    say(f"schedule outputs d={d} L={L} bq={bq} bk={bk} variant={variant} form={form}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    kr_gpu = None if kr is None else to_gpu(kr, torch.int32)
    bm, sched = va.blockmask_build(n_gpu, L, bq, bk, mask=m_gpu, key_range=kr_gpu, heads=H)
    g = [to_gpu_bf16(t) for t in (q, k, v, do)]
    kw = dict(block_mask=bm, mask=m_gpu, key_range=kr_gpu, bias=bias, variant=variant,
              block_q=bq, block_k=bk)
    res = []
    for s in (None, sched):
        o, lse = va.sigattn_fwd(*g[:3], n_gpu, return_lse=True, schedule=s, **kw)
        soft = dict(o=o, lse=lse) if variant != SIGMOID else {}
        grads = va.sigattn_bwd(*g, n_gpu, schedule=s, **soft, **kw)
        dk, dv = va.sigattn_bwd_dkdv(*g, n_gpu, schedule=s, **soft, **kw)
        dq = va.sigattn_bwd_dq(*g, n_gpu, schedule=s, **soft, **kw)
        out = [o, *grads, dk, dv, dq]
        if variant != SIGMOID:
            out.append(lse)
        res.append(out)
    torch.cuda.synchronize()
    for a, b_ in zip(*res):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                           b_.view(torch.int32) if b_.dtype == torch.float32 else b_.view(torch.int16))
    # The split halves equal the one-launch backward under the schedule too.
    assert torch.equal(res[1][2].view(torch.int16), res[1][4].view(torch.int16))
    assert torch.equal(res[1][1].view(torch.int16), res[1][6].view(torch.int16))


@pytest.mark.parametrize("form", ["none", "dense"])
def test_differential_identical_with_schedule(va, form):
    B, H, L, d = 5, 2, 270, 64
    n = np.array([270, 1, 0, 200, 129], np.int32)
    rng = np.random.default_rng(5)
    q1, k1, q2, k2, v, do = (syn.random_tensor(rng, (B, H, L, d)) for _ in range(6))
    m_gpu = None
    if form == "dense":
        m_gpu = to_gpu((rng.random((B, L, L)) < 0.5).astype(np.uint8), torch.uint8)
    say(f"schedule differential form={form}")
    n_gpu = to_gpu(n, torch.int32)
    bm, sched = va.blockmask_build(n_gpu, L, 64, 64, mask=m_gpu, heads=H)
    g = [to_gpu_bf16(t) for t in (q1, k1, q2, k2, v, do)]
    res = []
    for s in (None, sched):
        o, l1, l2, o1, o2 = va.sigattn_diff_fwd(*g[:5], n_gpu, 0.6, block_mask=bm, block_q=64,
                                                block_k=64, return_maps=True, schedule=s,
                                                mask=m_gpu)
        grads = va.sigattn_diff_bwd(*g, o1, o2, l1, l2, n_gpu, 0.6, block_mask=bm, block_q=64,
                                    block_k=64, schedule=s, mask=m_gpu)
        res.append([o, o1, o2, *grads])
    torch.cuda.synchronize()
    for a, b_ in zip(*res):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))


@pytest.mark.parametrize("variant,bias,d", [(SIGMOID, 1, 64), (SOFTMAX, 0, 64), (3, 0, 64),
                                            (SIGMOID, 1, 128), (3, 0, 128)])
def test_zero_items_write_every_padded_row(va, variant, bias, d):
    """With a schedule the fully padded tiles are zero items of their own, in
    runs of four 128-row tiles: L = 1100 (9 tiles) with n = 300 leaves tiles
    3..8 (a run of four, then of two), an empty sequence tiles 0..8 (runs of
    four, four and one).  Every output starts as NaN; with and without the
    schedule (forward, one-launch backward, its two halves, and differential
    attention, variant 3; at d = 128 its forward is two passes) the results
    are bit-identical, every padded row is +0 and every padded log-sum-exp
    -inf."""
    B, H, L = 3, 2, 1100
    n = np.array([L, 300, 0], np.int32)
    rng = np.random.default_rng(77 + variant)
    q, k, v, do, q2, k2 = (syn.random_tensor(rng, (B, H, L, d)) for _ in range(6))
    say(f"zero items variant={variant} d={d} L={L} n={n.tolist()}")
    n_gpu = to_gpu(n, torch.int32)
    bm, sched = va.blockmask_build(n_gpu, L, 128, 128, heads=H)
    g = [to_gpu_bf16(t) for t in (q, k, v, do, q2, k2)]

    def nan_like(t, dtype=None):
        return torch.full(t.shape if dtype is None else t.shape[:3], float("nan"),
                          dtype=dtype or t.dtype, device=t.device)

    res = []
    for s in (None, sched):
        if variant == 3:
            o, o1, o2 = (nan_like(g[0]) for _ in range(3))
            l1, l2 = nan_like(g[0], torch.float32), nan_like(g[0], torch.float32)
            va.sigattn_diff_fwd(g[0], g[1], g[4], g[5], g[2], n_gpu, 0.7, block_mask=bm,
                                schedule=s, out=o, o1=o1, o2=o2, lse1=l1, lse2=l2)
            grads = [nan_like(g[0]) for _ in range(5)]
            va.sigattn_diff_bwd(g[0], g[1], g[4], g[5], g[2], g[3], o1, o2, l1, l2, n_gpu, 0.7,
                                block_mask=bm, schedule=s, grads=grads)
            res.append([o, o1, o2, *grads, l1, l2])
            continue
        kw = dict(block_mask=bm, bias=bias, variant=variant, schedule=s)
        o = nan_like(g[0])
        lse = nan_like(g[0], torch.float32) if variant != SIGMOID else None
        va.sigattn_fwd(*g[:3], n_gpu, out=o, lse=lse, **kw)
        soft = dict(o=o, lse=lse) if variant != SIGMOID else {}
        dq, dk, dv, dk2, dv2, dq2 = (nan_like(g[0]) for _ in range(6))
        va.sigattn_bwd(*g[:4], n_gpu, dq=dq, dk=dk, dv=dv, **soft, **kw)
        va.sigattn_bwd_dkdv(*g[:4], n_gpu, dk=dk2, dv=dv2, **soft, **kw)
        va.sigattn_bwd_dq(*g[:4], n_gpu, dq=dq2, **soft, **kw)
        res.append([o, dq, dk, dv, dk2, dv2, dq2] + ([lse] if variant != SIGMOID else []))
    torch.cuda.synchronize()
    padded = torch.arange(L, device=n_gpu.device)[None, :] >= n_gpu[:, None]  # [B, L]
    for a, b_ in zip(*res):
        bits = (lambda t: t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16))
        assert torch.equal(bits(a), bits(b_))
        rows = padded[:, None, :].expand(B, H, L)
        if a.dtype == torch.float32:  # a log-sum-exp
            assert torch.all(torch.isneginf(a[rows]))
            assert not torch.isnan(a).any()
        else:
            assert torch.all(a.view(torch.int16)[rows] == 0), "a padded row is not +0"
            assert not torch.isnan(a.float()).any()
