"""Pins for the oracle's differential attention ("Differential Transformer"
note, "How differential attention works": two softmax maps over one V, the
second subtracted with a scalar lambda)."""
import numpy as np
import pytest

from _tiny import SOFTMAX, BIAS_NONE, dense_python, random_inputs, widen


@pytest.mark.parametrize("with_mask", [False, True])
def test_diff_matches_dense_two_maps(oracle_lib, with_mask):
    """Against two dense score matrices materialised in pure Python."""
    rng = np.random.default_rng(11)
    B, H, L, d = 2, 2, 14, 8
    q1, k1, q2, k2, v = random_inputs(rng, B, H, L, d, names="abcde")
    n = np.array([14, 9], np.int32)
    mask = (rng.random((B, L, L)) < 0.6).astype(np.uint8) if with_mask else None
    lam = 0.37
    o, lse1, lse2 = oracle_lib.diff_fwd(q1, k1, q2, k2, v, n, lam, mask=mask)
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(H):
            mb = None if mask is None else mask[b]
            w1 = dense_python(widen(q1[b, h]), widen(k1[b, h]), widen(v[b, h]), n[b], mb,
                              BIAS_NONE, SOFTMAX, scale)[1]
            w2 = dense_python(widen(q2[b, h]), widen(k2[b, h]), widen(v[b, h]), n[b], mb,
                              BIAS_NONE, SOFTMAX, scale)[1]
            want = (np.array(w1) - lam * np.array(w2)) @ widen(v[b, h])
            np.testing.assert_allclose(o[b, h], want, rtol=1e-12, atol=1e-13)


def test_identical_maps_scale_by_one_minus_lambda(oracle_lib):
    """Q2 = Q1 and K2 = K1: the two maps cancel to (1 - lambda) times one
    softmax attention; lambda = 1 gives exactly 0."""
    rng = np.random.default_rng(12)
    B, H, L, d = 2, 1, 40, 16
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([40, 23], np.int32)
    one, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX)
    for lam in (0.0, 0.8, 1.0, -0.5):
        o, l1, l2 = oracle_lib.diff_fwd(q, k, q, k, v, n, lam)
        np.testing.assert_allclose(o, (1 - lam) * one, rtol=1e-13, atol=1e-15)
        np.testing.assert_array_equal(l1, l2)
    o, _, _ = oracle_lib.diff_fwd(q, k, q, k, v, n, 1.0)
    assert np.all(o == 0)


def test_rows_match_full(oracle_lib):
    rng = np.random.default_rng(13)
    B, H, L, d = 2, 2, 30, 8
    q1, k1, q2, k2, v = random_inputs(rng, B, H, L, d, names="abcde")
    n = np.array([30, 17], np.int32)
    o, _, _ = oracle_lib.diff_fwd(q1, k1, q2, k2, v, n, 0.6)
    rows = [0, 5, 16, 29]
    got = oracle_lib.diff_fwd_rows(q1, k1, q2, k2, v, n, 0.6, 1, 1, rows)
    np.testing.assert_allclose(got, o[1, 1, rows], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("form", ["none", "mask", "range"])
def test_backward_rows_match_full(oracle_lib, form):
    """The sampled-row backward equals the rows of the whole-tensor backward
    (itself pinned by autograd below), with each mask form."""
    rng = np.random.default_rng(15)
    B, H, L, d = 2, 2, 30, 8
    q1, k1, q2, k2, v, do = random_inputs(rng, B, H, L, d, names="abcdef")
    n = np.array([30, 19], np.int32)
    mask = kr = None
    if form == "mask":
        mask = (rng.random((B, L, L)) < 0.5).astype(np.uint8)
    elif form == "range":
        lo = rng.integers(0, L, size=(B, L))
        kr = np.stack([lo, lo + rng.integers(-2, 12, size=(B, L))], axis=-1).astype(np.int32)
    lam = -0.7
    full = oracle_lib.diff_bwd(q1, k1, q2, k2, v, do, n, lam, mask=mask, key_range=kr)
    q_rows, k_rows = [0, 4, 18, 19, 29], [3, 4, 5, 17, 18, 19, 20]
    got = oracle_lib.diff_bwd_rows(q1, k1, q2, k2, v, do, n, lam, 1, 0, q_rows, k_rows,
                                   mask=mask, key_range=kr)
    for name, g_, f_ in zip(("dq1", "dk1", "dq2", "dk2", "dv"), got, full):
        rows = q_rows if name.startswith("dq") else k_rows
        np.testing.assert_allclose(g_, f_[1, 0, rows], rtol=1e-12, atol=1e-14, err_msg=name)


def test_diff_backward_matches_torch_autograd(oracle_lib):
    """Gradients of sum(dO * O) through two dense softmax maps, by torch float64
    autograd, against the oracle's composition."""
    import torch
    rng = np.random.default_rng(14)
    B, H, L, d = 2, 2, 12, 8
    q1, k1, q2, k2, v, do = random_inputs(rng, B, H, L, d, names="abcdef")
    n = np.array([12, 7], np.int32)
    mask = (rng.random((B, L, L)) < 0.5).astype(np.uint8)
    mask[:, np.arange(L), np.arange(L)] = 1  # every valid row sees a key
    lam = 0.45
    got = oracle_lib.diff_bwd(q1, k1, q2, k2, v, do, n, lam, mask=mask)
    t = [torch.tensor(widen(x), requires_grad=True) for x in (q1, k1, q2, k2, v)]
    tdo = torch.tensor(widen(do))
    idx = torch.arange(L)
    valid = (idx[None, :, None] < torch.tensor(n)[:, None, None]) & \
            (idx[None, None, :] < torch.tensor(n)[:, None, None]) & torch.tensor(mask != 0)
    row_ok = (idx[None, :] < torch.tensor(n)[:, None])[:, None, :, None]
    scale = 1.0 / np.sqrt(d)

    def probs(q, k):
        s = (q @ k.transpose(-1, -2)) * scale
        s = s.masked_fill(~valid[:, None], float("-inf"))
        return torch.where(row_ok, torch.softmax(s.masked_fill(~row_ok, 0.0), dim=-1), 0.0)

    o = (probs(t[0], t[1]) - lam * probs(t[2], t[3])) @ t[4]
    (o * tdo * row_ok).sum().backward()
    for name, g_, tt in zip(("dq1", "dk1", "dq2", "dk2", "dv"), got, t):
        np.testing.assert_allclose(g_, tt.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)
