"""sigattn_fwd_noalloc (the forward with its work schedule in the library's
own device memory, for callers that cannot allocate) against the existing
entry point it varies, sigattn_fwd with a schedule from blockmask_build:
through the C ABI, three calls in a row, each smaller than the one before
(padding only, a dense mask, key ranges), each bit for bit equal to
sigattn_fwd's result and within the parity bounds of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from _gpu import assert_rows, gpu_f64, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

SIGMOID, SOFTMAX = 0, 1


@pytest.fixture(scope="module")
def va():
    import varlen_attention_amd as va
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    va.load_library()
    return va


def _case(va, seed, B, H, L, d, n, variant, bias, block, form):
    """form: "none" (padding only), "dense" (a [B, L, L] element mask) or
    "range" (inclusive key ranges [B, L, 2]: causal windows of random width,
    one row empty)."""
    rng = np.random.default_rng(seed)
    q, k, v = (syn.random_tensor(rng, (B, H, L, d)) for _ in range(3))
    mask = kr = None
    if form == "dense":
        mask = (rng.random((B, L, L)) < 0.4).astype(np.uint8)
        mask[0, 2, :] = 0
    elif form == "range":
        r = np.arange(L)
        kr = np.stack([r[None, :] - rng.integers(0, 40, size=(B, L)),
                       np.broadcast_to(r, (B, L))], axis=2).astype(np.int32)
        kr[0, 1] = (5, 1)  # empty
    say(f"no-alloc forward B={B} H={H} L={L} d={d} variant={variant} form={form}")
    n_gpu = to_gpu(n, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    kr_gpu = None if kr is None else to_gpu(kr, torch.int32)
    g = [to_gpu_bf16(t) for t in (q, k, v)]
    kw = dict(mask=m_gpu, key_range=kr_gpu, bias=bias, variant=variant, block_q=block,
              block_k=block)
    bm, sched = va.blockmask_build(n_gpu, L, block, block, mask=m_gpu, key_range=kr_gpu,
                                   heads=H)
    o_ref, lse_ref = va.sigattn_fwd(*g, n_gpu, block_mask=bm, schedule=sched, return_lse=True,
                                    **kw)
    o = torch.empty_like(g[0])
    lse = torch.empty((B, H, L), dtype=torch.float32, device=g[0].device)
    va.sigattn_fwd_noalloc(*g, n_gpu, bm, o, lse=lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    if variant != SIGMOID:
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32))
    want, _ = oracle.fwd(q, k, v, n, mask=mask, key_range=kr, bias=bias, variant=variant)
    assert_rows(gpu_f64(o), want, n, "O (no-alloc)")


def test_noalloc_forward_twice_second_smaller(va):
    _case(va, 11, 6, 3, 300, 64, np.array([300, 211, 1, 0, 128, 299], np.int32), SIGMOID, 1, 128,
          "none")
    _case(va, 12, 3, 2, 150, 128, np.array([150, 77, 0], np.int32), SOFTMAX, 0, 64, "dense")
    _case(va, 13, 2, 2, 100, 64, np.array([100, 61], np.int32), SOFTMAX, 0, 32, "range")
