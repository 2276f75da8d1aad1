"""Pins for the oracle's backward pass (dQ, dK, dV).

The oracle writes the gradients out by hand (sigmoid: diagonal Jacobian
sigma (1 - sigma), single-cell page section 2.B; softmax family: p (dp - D)).
These tests fix them to independent derivations: central finite differences
of the pure-Python forward, torch CPU float64 autograd of the dense masked
expression, the inner-product identities <dQ,Q> = <dK,K> and <dV,V> = <dO,O>,
and the bound sigma' <= 1/4 stated by the page."""
import numpy as np
import pytest
import scipy.special
import torch

from _tiny import (BIAS_LOG_PADLEN, BIAS_LOG_SEQLEN, BIAS_NONE, SIGMOID, SOFTMAX, SOFTMAX1,
                   bf16, dense_python, random_inputs, widen)

VARIANTS = [SIGMOID, SOFTMAX, SOFTMAX1]


def loss_python(qf, kf, vf, dof, n, mask_b, bias, variant, scale):
    o, _ = dense_python(qf, kf, vf, n, mask_b, bias, variant, scale)
    return float((o * dof).sum())


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("with_mask", [False, True])
def test_finite_differences(oracle_lib, variant, with_mask):
    rng = np.random.default_rng(200 + variant + 10 * with_mask)
    L, d = 6, 4
    q, k, v, do = random_inputs(rng, 1, 1, L, d, names="qkvd")
    n = 5
    mask = (rng.random((1, L, L)) < 0.7).astype(np.uint8) if with_mask else None
    bias = BIAS_LOG_SEQLEN if variant == SIGMOID else BIAS_NONE
    scale = 0.6
    dq, dk, dv = oracle_lib.bwd(q, k, v, do, np.array([n], np.int32), mask=mask, bias=bias,
                                variant=variant, scale=scale)
    base = [widen(t[0, 0]) for t in (q, k, v)]
    dof = widen(do[0, 0])
    mb = None if mask is None else mask[0]
    eps = 1e-6
    for which, grad in enumerate((dq, dk, dv)):
        fd = np.zeros((L, d))
        for r in range(L):
            for t in range(d):
                args_p = [x.copy() for x in base]
                args_m = [x.copy() for x in base]
                args_p[which][r, t] += eps
                args_m[which][r, t] -= eps
                fp = loss_python(*args_p, dof, n, mb, bias, variant, scale)
                fm = loss_python(*args_m, dof, n, mb, bias, variant, scale)
                fd[r, t] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(grad[0, 0], fd, rtol=1e-6, atol=1e-8)


def torch_dense_loss(q, k, v, do, valid, beta, variant, scale):
    s = scale * (q @ k.transpose(-1, -2)) + beta
    if variant == SIGMOID:
        p = torch.where(valid, torch.sigmoid(s), torch.zeros_like(s))
    else:
        neg = torch.full_like(s, -torch.inf)
        sm = torch.where(valid, s, neg)
        m = sm.amax(dim=-1, keepdim=True).detach()
        if variant == SOFTMAX1:
            m = torch.clamp(m, min=0.0)
        m = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
        e = torch.where(valid, torch.exp(s - m), torch.zeros_like(s))
        denom = e.sum(-1, keepdim=True)
        if variant == SOFTMAX1:
            denom = denom + torch.exp(-m)
        denom = torch.where(denom > 0, denom, torch.ones_like(denom))
        p = e / denom
    return ((p @ v) * do).sum()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("bias", [BIAS_NONE, BIAS_LOG_SEQLEN, BIAS_LOG_PADLEN])
def test_matches_torch_autograd(oracle_lib, variant, bias):
    rng = np.random.default_rng(300 + variant * 3 + bias)
    B, H, L, d = 3, 2, 37, 16
    q, k, v, do = random_inputs(rng, B, H, L, d, names="qkvd")
    n = np.array([37, 20, 3], np.int32)
    mask = (rng.random((B, L, L)) < 0.6).astype(np.uint8)
    mask[1, 4, :] = 0  # a valid query row with no valid key
    dq, dk, dv = oracle_lib.bwd(q, k, v, do, n, mask=mask, bias=bias, variant=variant)
    idx = np.arange(L)
    scale = 1 / 4
    for b in range(B):
        nb = int(n[b])
        valid = torch.from_numpy((idx[:, None] < nb) & (idx[None, :] < nb) & (mask[b] != 0))
        beta = {BIAS_NONE: 0.0, BIAS_LOG_SEQLEN: -np.log(nb), BIAS_LOG_PADLEN: -np.log(L)}[bias]
        for h in range(H):
            tq, tk, tv = (torch.from_numpy(widen(t[b, h])).requires_grad_() for t in (q, k, v))
            tdo = torch.from_numpy(widen(do[b, h]))
            torch_dense_loss(tq, tk, tv, tdo, valid, beta, variant, scale).backward()
            np.testing.assert_allclose(dq[b, h], tq.grad.numpy(), rtol=1e-9, atol=1e-12)
            np.testing.assert_allclose(dk[b, h], tk.grad.numpy(), rtol=1e-9, atol=1e-12)
            np.testing.assert_allclose(dv[b, h], tv.grad.numpy(), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("variant", VARIANTS)
def test_inner_product_identities(oracle_lib, variant):
    """s depends on q and k only through scale * <q, k>: <dQ,Q> = <dK,K>;
    o is linear in v: <dV,V> = <dO,O>."""
    rng = np.random.default_rng(400 + variant)
    B, H, L, d = 2, 2, 70, 32
    q, k, v, do = random_inputs(rng, B, H, L, d, names="qkvd")
    n = np.array([70, 41], np.int32)
    bias = BIAS_LOG_SEQLEN if variant == SIGMOID else BIAS_NONE
    dq, dk, dv = oracle_lib.bwd(q, k, v, do, n, bias=bias, variant=variant)
    o, _ = oracle_lib.fwd(q, k, v, n, bias=bias, variant=variant)
    qf, kf, vf, dof = (widen(t) for t in (q, k, v, do))
    for b in range(B):
        for h in range(H):
            a, c = (dq[b, h] * qf[b, h]).sum(), (dk[b, h] * kf[b, h]).sum()
            assert abs(a - c) <= 1e-10 * max(1.0, abs(a))
            nb = n[b]
            e, f = (dv[b, h] * vf[b, h]).sum(), (dof[b, h, :nb] * o[b, h, :nb]).sum()
            assert abs(e - f) <= 1e-10 * max(1.0, abs(e))


def test_sigmoid_derivative_bound(oracle_lib):
    """K = identity rows, V_c = e_0, dO_r = e_0: dP = 1, so dQ_r[c] = scale * sigma'(s)
    with sigma' = sigma (1 - sigma) <= 1/4, reached at s = 0."""
    L, d, n = 16, 16, 16
    qv = np.linspace(-12, 12, L * d).reshape(L, d)
    qv[3, 5] = 0.0
    eye = np.eye(L, d)
    e0 = np.zeros((L, d))
    e0[:, 0] = 1
    q, k, v, do = (bf16(x)[None, None] for x in (qv, eye, e0, e0))
    scale = 1.0
    dq, _, _ = oracle_lib.bwd(q, k, v, do, np.array([n], np.int32), bias=BIAS_NONE,
                              variant=SIGMOID, scale=scale)
    s = widen(q[0, 0])[:, :L]
    sig = scipy.special.expit(s)
    np.testing.assert_allclose(dq[0, 0, :, :L], sig * (1 - sig), rtol=1e-12, atol=1e-300)
    assert dq.max() <= 0.25 and dq[0, 0, 3, 5] == 0.25


def test_softmax_score_gradients_sum_to_zero(oracle_lib):
    """Softmax is unchanged by a shift of a row, so each row of dS sums to 0;
    softmax_1 is not shift-invariant and its rows do not."""
    rng = np.random.default_rng(500)
    L, d, n = 12, 12, 12
    qv = rng.standard_normal((L, d)) * 2
    eye = np.eye(L, d)
    q, k = bf16(qv)[None, None], bf16(eye)[None, None]
    v, do = (bf16(rng.standard_normal((1, 1, L, d))) for _ in range(2))
    dq, _, _ = oracle_lib.bwd(q, k, v, do, np.array([n], np.int32), bias=BIAS_NONE,
                              variant=SOFTMAX, scale=1.0)
    np.testing.assert_allclose(dq[0, 0].sum(axis=1), 0.0, atol=1e-13)
    dq1, _, _ = oracle_lib.bwd(q, k, v, do, np.array([n], np.int32), bias=BIAS_NONE,
                               variant=SOFTMAX1, scale=1.0)
    assert np.abs(dq1[0, 0].sum(axis=1)).max() > 1e-6


@pytest.mark.parametrize("variant", VARIANTS)
def test_padding_zero_and_poison_ignored(oracle_lib, variant):
    rng = np.random.default_rng(600 + variant)
    B, H, L, d = 2, 1, 45, 8
    q, k, v, do = random_inputs(rng, B, H, L, d, names="qkvd")
    n = np.array([29, 45], np.int32)
    g = oracle_lib.bwd(q, k, v, do, n, variant=variant)
    poisoned = [t.copy() for t in (q, k, v, do)]
    for t in poisoned:
        t[0, :, n[0]:] = np.uint16(0x7FC0)
    gp = oracle_lib.bwd(*poisoned, n, variant=variant)
    for a, b in zip(g, gp):
        assert np.array_equal(a, b)
        assert np.all(a[0, :, n[0]:] == 0)


def test_fp32_statement_agrees_with_fp64(oracle_lib):
    rng = np.random.default_rng(700)
    B, H, L, d = 1, 2, 200, 64
    q, k, v, do = random_inputs(rng, B, H, L, d, names="qkvd")
    n = np.array([190], np.int32)
    g64 = oracle_lib.bwd(q, k, v, do, n, precision="f64")
    g32 = oracle_lib.bwd(q, k, v, do, n, precision="f32")
    for a, b in zip(g64, g32):
        assert np.linalg.norm(a - b) / np.linalg.norm(a) < 1e-5


def test_rows_api_matches_full(oracle_lib):
    rng = np.random.default_rng(800)
    B, H, L, d = 2, 1, 33, 8
    q, k, v, do = random_inputs(rng, B, H, L, d, names="qkvd")
    n = np.array([33, 14], np.int32)
    for variant in VARIANTS:
        dq, dk, dv = oracle_lib.bwd(q, k, v, do, n, variant=variant)
        rows = [0, 7, 13, 14, 32]
        rq, rk, rv = oracle_lib.bwd_rows(q, k, v, do, n, 1, 0, rows, rows, variant=variant)
        assert np.array_equal(rq, dq[1, 0, rows])
        assert np.array_equal(rk, dk[1, 0, rows]) and np.array_equal(rv, dv[1, 0, rows])


@pytest.mark.parametrize("variant", [SOFTMAX, SOFTMAX1])
def test_given_output_shifts_only_D(oracle_lib, variant):
    """The softmax-family backward handed a stored output o forms
    D_r = <dO_r, o_r> from it.  Changing D by delta_r changes dS[r, c] by
    -P[r, c] delta_r, so, against the exact output: dQ_r moves by
    -scale delta_r sum_c P[r, c] k_c, dK_c by -scale sum_r P[r, c] delta_r q_r,
    and dV not at all (P from the dense pure-Python reference)."""
    from _tiny import dense_python, random_inputs, widen
    rng = np.random.default_rng(17 + variant)
    B, H, L, d = 2, 1, 7, 4
    q, k, v, do = random_inputs(rng, B, H, L, d, names="qkvd")
    n = np.array([7, 4], np.int32)
    mask = (rng.random((B, L, L)) < 0.7).astype(np.uint8)
    scale = 0.6
    o_exact, _ = oracle_lib.fwd(q, k, v, n, mask=mask, bias=0, variant=variant, scale=scale)
    o_given = bf16(o_exact + 0.05 * rng.standard_normal(o_exact.shape))  # any stored output
    g_exact = oracle_lib.bwd(q, k, v, do, n, mask=mask, bias=0, variant=variant, scale=scale)
    g_given = oracle_lib.bwd(q, k, v, do, n, mask=mask, bias=0, variant=variant, scale=scale,
                             o=o_given)
    np.testing.assert_array_equal(g_given[2], g_exact[2])  # dV
    qf, kf, vf, dof, of = (widen(t) for t in (q, k, v, do, o_given))
    for b in range(B):
        _, P = dense_python(qf[b, 0], kf[b, 0], vf[b, 0], n[b], mask[b], 0, variant, scale)
        delta = (dof[b, 0] * of[b, 0]).sum(1) - (dof[b, 0] * o_exact[b, 0]).sum(1)
        delta[int(n[b]):] = 0.0
        want_dq = g_exact[0][b, 0] - scale * delta[:, None] * (P @ kf[b, 0])
        want_dk = g_exact[1][b, 0] - scale * (P * delta[:, None]).T @ qf[b, 0]
        np.testing.assert_allclose(g_given[0][b, 0], want_dq, rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(g_given[1][b, 0], want_dk, rtol=1e-9, atol=1e-11)


def test_given_exact_output_changes_nothing_in_sigmoid(oracle_lib):
    """SIGMOID has no D: a given output is ignored."""
    from _tiny import random_inputs
    rng = np.random.default_rng(3)
    q, k, v, do = random_inputs(rng, 1, 2, 9, 8, names="qkvd")
    n = np.array([9], np.int32)
    a = oracle_lib.bwd(q, k, v, do, n, variant=SIGMOID)
    b_ = oracle_lib.bwd(q, k, v, do, n, variant=SIGMOID, o=v)
    for x, y in zip(a, b_):
        np.testing.assert_array_equal(x, y)
