"""Complete GPU parity at the benchmark workloads' full sizes: every valid row
of every output (O, LSE, dQ, dK, dV) against the fp64 oracle on the same
seeded bf16 inputs, in the launch configurations the benchmark times.

Workloads (seed 0, from ``synthetic``):
* single cell, B32 H8 d64, log-normal lengths (median 800) padded to the
  batch maximum L = 1584: sigmoid with the -ln n bias at block 128 (the
  benchmark's step) and block 64, and the softmax and softmax_1 variants
  (forward and backward, no bias);
* long packed documents, B8 H16 d128, L = 7122, causal mask within
  documents (dense [B, L, L] form), block 128, sigmoid with -ln n;
* differential attention at the single-cell shapes (lambda 0.8).

Bounds: per element |got - want| <= 1e-2 max(1, |want|), relative L2 <=
5e-3 over the valid rows, padded rows exactly zero, block masks bit for bit.

With SIGATTN_PARITY_LOG=<path> each comparison also appends one JSON line
(workload, variant, direction, output, max-abs figure, relative L2, oracle
seconds) to that file; the benchmark's measurement suite attaches these
errors to its rows."""
import json
import os
import time

import numpy as np
import pytest
import torch

import oracle
import synthetic as syn
from _gpu import assert_rows, gpu_f64, row_valid, say, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

SIGMOID, SOFTMAX, SOFTMAX1 = 0, 1, 2
VARIANT_NAMES = {SIGMOID: "sigmoid", SOFTMAX: "softmax", SOFTMAX1: "softmax_1"}


@pytest.fixture(scope="module")
def va():
    import varlen_attention_amd as va
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    va.load_library()
    return va


@pytest.fixture(scope="module")
def single_cell():
    return syn.single_cell_backward(0)  # the forward workload's lengths and tensors, plus dO


@pytest.fixture(scope="module")
def single_cell_sigmoid_ref(single_cell):
    """The oracle's sigmoid (-ln n) forward and backward over all 256
    (batch entry, head) pairs, shared by the block-128 and block-64 tests."""
    w = single_cell
    t0 = time.perf_counter()
    o, _ = oracle.fwd(w.q, w.k, w.v, w.seq_lens, bias=1, variant=SIGMOID)
    t1 = time.perf_counter()
    grads = oracle.bwd(w.q, w.k, w.v, w.do, w.seq_lens, bias=1, variant=SIGMOID)
    t2 = time.perf_counter()
    return {"O": o, "dQ": grads[0], "dK": grads[1], "dV": grads[2],
            "fwd_s": t1 - t0, "bwd_s": t2 - t1}


def _log(w, variant, direction, output, res, oracle_s, mask="none", **extra):
    path = os.environ.get("SIGATTN_PARITY_LOG")
    if not path:
        return
    rec = {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "variant": variant,
           "direction": direction, "output": output, "mask": mask, "max_abs": res[0],
           "rel_l2": res[1], "oracle_s": round(oracle_s, 2), **extra}
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def _run_gpu(va, w, variant, bias, block, mask=None):
    """Block mask and schedule, forward (with LSE for the softmax variants) and
    backward through the C ABI, as the benchmark launches them."""
    n_gpu = to_gpu(w.seq_lens, torch.int32)
    m_gpu = None if mask is None else to_gpu(mask, torch.uint8)
    bm, sched = va.blockmask_build(n_gpu, w.L, block, block, mask=m_gpu, heads=w.H)
    q, k, v, do = (to_gpu_bf16(t) for t in (w.q, w.k, w.v, w.do))
    kw = dict(block_mask=bm, schedule=sched, mask=m_gpu, bias=bias, variant=variant,
              block_q=block, block_k=block)
    if variant == SIGMOID:
        o, lse = va.sigattn_fwd(q, k, v, n_gpu, **kw), None
        dq, dk, dv = va.sigattn_bwd(q, k, v, do, n_gpu, **kw)
    else:
        o, lse = va.sigattn_fwd(q, k, v, n_gpu, return_lse=True, **kw)
        dq, dk, dv = va.sigattn_bwd(q, k, v, do, n_gpu, o=o, lse=lse, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bm.cpu().numpy(),
                                  oracle.blockmask(w.seq_lens, mask, w.L, block, block))
    out = {"O": gpu_f64(o), "dQ": gpu_f64(dq), "dK": gpu_f64(dk), "dV": gpu_f64(dv)}
    if lse is not None:
        out["LSE"] = lse.cpu().numpy().astype(np.float64)
    return out


def _check_lse(got, want, seq_lens, what):
    """LSE of valid rows within 1e-3 max(1, |want|); -inf exactly where the
    oracle has it (rows without a valid key) and on every padded row."""
    B, H, L = got.shape
    valid = np.broadcast_to(row_valid(seq_lens, B, L)[:, None, :], (B, H, L))
    assert np.all(np.isneginf(got[~valid])), f"{what}: padded LSE not -inf"
    g, w_ = got[valid], want[valid]
    assert np.array_equal(np.isneginf(g), np.isneginf(w_)), f"{what}: -inf rows differ"
    fin = np.isfinite(w_)
    err = float((np.abs(g[fin] - w_[fin]) / np.maximum(1.0, np.abs(w_[fin]))).max())
    assert err <= 1e-3, f"{what}: LSE error {err:.3e}"
    return err


@pytest.mark.parametrize("block", [128, 64])
def test_single_cell_sigmoid_complete(va, single_cell, single_cell_sigmoid_ref, block):
    """The benchmark's step (block 128) and the 64-block launch: every valid
    row of O, dQ, dK, dV of all 256 (batch entry, head) pairs."""
    w, ref = single_cell, single_cell_sigmoid_ref
    say(f"single cell complete sigmoid block={block} L={w.L}")
    got = _run_gpu(va, w, SIGMOID, 1, block)
    for name in ("O", "dQ", "dK", "dV"):
        res = assert_rows(got[name], ref[name], w.seq_lens, f"single cell block {block} {name}")
        _log(w, "sigmoid", "fwd" if name == "O" else "bwd", name, res,
             ref["fwd_s" if name == "O" else "bwd_s"], block=block)
        say(f"  {name}: max abs {res[0]:.3e} rel L2 {res[1]:.3e}")


@pytest.mark.parametrize("variant", [SOFTMAX, SOFTMAX1])
def test_single_cell_softmax_family_complete(va, single_cell, variant):
    """Online softmax and softmax_1 through the same tile loop at the
    single-cell shapes (no bias): every valid row of O, LSE and the
    gradients (backward from the forward's O and LSE)."""
    w = single_cell
    say(f"single cell complete variant={variant}")
    got = _run_gpu(va, w, variant, 0, 128)
    t0 = time.perf_counter()
    o, lse = oracle.fwd(w.q, w.k, w.v, w.seq_lens, bias=0, variant=variant)
    t1 = time.perf_counter()
    dq, dk, dv = oracle.bwd(w.q, w.k, w.v, w.do, w.seq_lens, bias=0, variant=variant)
    t2 = time.perf_counter()
    vname = VARIANT_NAMES[variant]
    err = _check_lse(got["LSE"], lse, w.seq_lens, f"{vname} LSE")
    say(f"  LSE: max error {err:.3e}")
    for name, want, dt in (("O", o, t1 - t0), ("dQ", dq, t2 - t1), ("dK", dk, t2 - t1),
                           ("dV", dv, t2 - t1)):
        res = assert_rows(got[name], want, w.seq_lens, f"single cell {vname} {name}")
        _log(w, vname, "fwd" if name == "O" else "bwd", name, res, dt, block=128)
        say(f"  {name}: max abs {res[0]:.3e} rel L2 {res[1]:.3e}")


def test_long_documents_complete(va):
    """Long packed documents (B8 H16 d128, L 7122, causal within documents,
    dense mask, block 128): every valid row of O, dQ, dK, dV."""
    w = syn.long_packed_docs(0, tensors=("q", "k", "v", "do"))
    say(f"long documents complete L={w.L}")
    got = _run_gpu(va, w, SIGMOID, 1, 128, mask=w.mask)
    t0 = time.perf_counter()
    o, _ = oracle.fwd(w.q, w.k, w.v, w.seq_lens, mask=w.mask, bias=1, variant=SIGMOID)
    t1 = time.perf_counter()
    dq, dk, dv = oracle.bwd(w.q, w.k, w.v, w.do, w.seq_lens, mask=w.mask, bias=1,
                            variant=SIGMOID)
    t2 = time.perf_counter()
    for name, want, dt in (("O", o, t1 - t0), ("dQ", dq, t2 - t1), ("dK", dk, t2 - t1),
                           ("dV", dv, t2 - t1)):
        res = assert_rows(got[name], want, w.seq_lens, f"long documents {name}")
        _log(w, "sigmoid", "fwd" if name == "O" else "bwd", name, res, dt, mask="dense",
             block=128)
        say(f"  {name}: max abs {res[0]:.3e} rel L2 {res[1]:.3e}")


def test_differential_single_cell_complete(va, single_cell):
    """Differential attention at the single-cell shapes (lambda 0.8, block
    128): every valid row of O, both LSEs and all five gradients."""
    w = single_cell
    rng = np.random.default_rng(21)
    q2 = syn.random_tensor(rng, w.q.shape)
    k2 = syn.random_tensor(rng, w.k.shape)
    lam = 0.8
    say(f"differential complete L={w.L}")
    n_gpu = to_gpu(w.seq_lens, torch.int32)
    bm, sched = va.blockmask_build(n_gpu, w.L, 128, 128, heads=w.H)
    g = [to_gpu_bf16(t) for t in (w.q, w.k, q2, k2, w.v, w.do)]
    o, l1, l2, o1, o2 = va.sigattn_diff_fwd(*g[:5], n_gpu, lam, return_maps=True,
                                            block_mask=bm, schedule=sched)
    grads = va.sigattn_diff_bwd(*g, o1, o2, l1, l2, n_gpu, lam, block_mask=bm, schedule=sched)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    want_o, want_l1, want_l2 = oracle.diff_fwd(w.q, w.k, q2, k2, w.v, w.seq_lens, lam)
    t1 = time.perf_counter()
    want_g = oracle.diff_bwd(w.q, w.k, q2, k2, w.v, w.do, w.seq_lens, lam)
    t2 = time.perf_counter()
    for got_l, want_l, nm in ((l1, want_l1, "LSE1"), (l2, want_l2, "LSE2")):
        _check_lse(got_l.cpu().numpy().astype(np.float64), want_l, w.seq_lens, nm)
    res = assert_rows(gpu_f64(o), want_o, w.seq_lens, "differential O")
    _log(w, "differential", "fwd", "O", res, t1 - t0, block=128, lam=lam)
    for name, got_t, want in zip(("dQ1", "dK1", "dQ2", "dK2", "dV"), grads, want_g):
        res = assert_rows(gpu_f64(got_t), want, w.seq_lens, f"differential {name}")
        _log(w, "differential", "bwd", name, res, t2 - t1, block=128, lam=lam)
        say(f"  {name}: max abs {res[0]:.3e} rel L2 {res[1]:.3e}")
