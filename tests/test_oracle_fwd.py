"""Pins for the oracle's forward pass.

Each test fixes the oracle to something other than itself: a pure-Python
dense computation on tiny inputs, closed forms, library routines (torch CPU
scaled_dot_product_attention, scipy's softmax and expit) on special inputs,
and invariants stated by the pages (row sums, softmax_1 limits and ratios,
the zero-logit equivalence of softmax_1, permutation of keys, block
skipping)."""
import os

import numpy as np
import pytest
import scipy.special
import torch

from _tiny import (BIAS_LOG_PADLEN, BIAS_LOG_SEQLEN, BIAS_NONE, SIGMOID, SOFTMAX, SOFTMAX1,
                   bf16, dense_python, random_inputs, widen)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
VARIANTS = [SIGMOID, SOFTMAX, SOFTMAX1]
BIASES = [BIAS_NONE, BIAS_LOG_SEQLEN, BIAS_LOG_PADLEN]


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(x) for x in line.split()])
    return np.array(rows)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("bias", BIASES)
@pytest.mark.parametrize("with_mask", [False, True])
def test_matches_python_bruteforce(oracle_lib, variant, bias, with_mask):
    rng = np.random.default_rng(100 + 10 * variant + bias + 50 * with_mask)
    B, H, L, d = 3, 2, 9, 5
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([9, 4, 1], dtype=np.int32)
    mask = (rng.random((B, L, L)) < 0.6).astype(np.uint8) if with_mask else None
    if with_mask:
        mask[0, 2, :] = 0  # a valid query row with no valid key
    scale = 0.37
    o, lse = oracle_lib.fwd(q, k, v, n, mask=mask, bias=bias, variant=variant, scale=scale)
    for b in range(B):
        for h in range(H):
            want, _ = dense_python(widen(q[b, h]), widen(k[b, h]), widen(v[b, h]), n[b],
                                   None if mask is None else mask[b], bias, variant, scale)
            np.testing.assert_allclose(o[b, h], want, rtol=1e-12, atol=1e-13)


def onehot_inputs(rng, L, d, q_values):
    """K = V = identity rows (d >= L): scores become scale * Q[:, :L] + beta and
    the output's first L columns are the attention weights themselves."""
    eye = np.zeros((L, d), dtype=np.float32)
    eye[np.arange(L), np.arange(L)] = 1.0
    q = bf16(q_values)[None, None]
    k = bf16(eye)[None, None]
    v = bf16(eye)[None, None]
    return q, k, v


@pytest.mark.parametrize("bias", BIASES)
def test_sigmoid_weights_are_expit_of_scores(oracle_lib, bias):
    rng = np.random.default_rng(1)
    L, d, n = 12, 16, 10
    qv = rng.standard_normal((L, d)) * 3
    q, k, v = onehot_inputs(rng, L, d, qv)
    scale = 0.25
    o, _ = oracle_lib.fwd(q, k, v, np.array([n], np.int32), bias=bias, variant=SIGMOID,
                          scale=scale)
    beta = {BIAS_NONE: 0.0, BIAS_LOG_SEQLEN: -np.log(n), BIAS_LOG_PADLEN: -np.log(L)}[bias]
    s = scale * widen(q[0, 0])[:n, :n] + beta
    np.testing.assert_allclose(o[0, 0, :n, :n], scipy.special.expit(s), rtol=1e-13)
    assert np.all(o[0, 0, :n, n:] == 0) and np.all(o[0, 0, n:] == 0)


@pytest.mark.parametrize("variant", [SOFTMAX, SOFTMAX1])
def test_softmax_weights_and_lse_are_library_softmax(oracle_lib, variant):
    rng = np.random.default_rng(2)
    L, d, n = 12, 16, 11
    qv = rng.standard_normal((L, d)) * 4
    q, k, v = onehot_inputs(rng, L, d, qv)
    scale = 0.5
    o, lse = oracle_lib.fwd(q, k, v, np.array([n], np.int32), bias=BIAS_NONE, variant=variant,
                            scale=scale)
    s = scale * widen(q[0, 0])[:n, :n]
    if variant == SOFTMAX:
        want = scipy.special.softmax(s, axis=1)
        want_lse = scipy.special.logsumexp(s, axis=1)
    else:  # softmax_1 = softmax over the logits plus one extra zero logit
        ext = np.concatenate([np.zeros((n, 1)), s], axis=1)
        want = scipy.special.softmax(ext, axis=1)[:, 1:]
        want_lse = scipy.special.logsumexp(ext, axis=1)
    np.testing.assert_allclose(o[0, 0, :n, :n], want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, :n], want_lse, rtol=1e-13)
    assert np.all(np.isneginf(lse[0, 0, n:]))


def test_sigmoid_closed_form_with_zero_queries(oracle_lib):
    """Q = 0 and bias -ln n: o_r = sum_{c<n} v_c / (1 + n) for every valid row."""
    rng = np.random.default_rng(3)
    B, H, L, d = 4, 2, 40, 8
    _, k, v = random_inputs(rng, B, H, L, d)
    q = np.zeros_like(k)
    n = np.array([40, 17, 1, 3], dtype=np.int32)
    o, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_LOG_SEQLEN, variant=SIGMOID)
    for b in range(B):
        for h in range(H):
            want = widen(v[b, h])[: n[b]].sum(axis=0) / (1 + n[b])
            np.testing.assert_allclose(o[b, h, : n[b]], np.broadcast_to(want, (n[b], d)),
                                       rtol=1e-13, atol=1e-15)
            assert np.all(o[b, h, n[b]:] == 0)


def test_sigmoid_bias_golden_values(oracle_lib):
    """Q = 0, V = 1: every element equals n / (n + 1) (golden fixture)."""
    table = read_golden("sigmoid_bias_closed_form.txt")
    for n_val, sig, elem in table:
        n = int(n_val)
        assert abs(1.0 / (1.0 + n) - sig) < 1e-15
        L, d = max(n, 2), 4
        q = np.zeros((1, 1, L, d), dtype=np.uint16)
        k = bf16(np.random.default_rng(n).standard_normal((1, 1, L, d)))
        v = bf16(np.ones((1, 1, L, d)))
        o, _ = oracle_lib.fwd(q, k, v, np.array([n], np.int32), bias=BIAS_LOG_SEQLEN,
                              variant=SIGMOID)
        np.testing.assert_allclose(o[0, 0, :n], elem, rtol=1e-14)


def test_single_key_sequence(oracle_lib):
    """n = 1: beta = -ln 1 = 0, so o_0 = sigma(scale q_0.k_0) v_0 (sigmoid) and v_0 (softmax)."""
    rng = np.random.default_rng(4)
    L, d = 8, 16
    q, k, v = random_inputs(rng, 1, 1, L, d)
    n = np.array([1], np.int32)
    scale = 1 / 4
    qf, kf, vf = widen(q[0, 0]), widen(k[0, 0]), widen(v[0, 0])
    o, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_LOG_SEQLEN, variant=SIGMOID, scale=scale)
    s = scale * float(qf[0] @ kf[0])
    np.testing.assert_allclose(o[0, 0, 0], scipy.special.expit(s) * vf[0], rtol=1e-13)
    o, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX, scale=scale)
    np.testing.assert_allclose(o[0, 0, 0], vf[0], rtol=1e-14)
    assert np.all(o[0, 0, 1:] == 0)


@pytest.mark.parametrize("with_mask", [False, True])
def test_softmax_matches_torch_sdpa(oracle_lib, with_mask):
    rng = np.random.default_rng(5)
    B, H, L, d = 3, 2, 33, 16
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([33, 20, 7], dtype=np.int32)
    mask = (rng.random((B, L, L)) < 0.5).astype(np.uint8) if with_mask else None
    o, lse = oracle_lib.fwd(q, k, v, n, mask=mask, bias=BIAS_NONE, variant=SOFTMAX)
    idx = np.arange(L)
    valid = (idx[None, :, None] < n[:, None, None]) & (idx[None, None, :] < n[:, None, None])
    if mask is not None:
        valid &= mask != 0
    tq, tk, tv = (torch.from_numpy(widen(t)) for t in (q, k, v))
    attn_mask = torch.from_numpy(valid)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn_mask)
    has_key = valid.any(axis=2)
    for b in range(B):
        for h in range(H):
            rows = has_key[b]
            np.testing.assert_allclose(o[b, h, rows], ref[b, h, rows].numpy(), rtol=1e-10,
                                       atol=1e-12)
            assert np.all(o[b, h, ~rows] == 0) and np.all(np.isneginf(lse[b, h, ~rows]))


def test_softmax1_equals_softmax_with_prepended_zero_key(oracle_lib):
    """softmax_1 page, "Properties" and comments: prepending a zero key with a
    zero value adds 1 to every denominator."""
    rng = np.random.default_rng(6)
    B, H, L, d = 2, 3, 25, 8
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([25, 9], dtype=np.int32)
    o1, lse1 = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX1)
    # Library check: torch SDPA over n + 1 keys, the first one zero.
    tq, tk, tv = (torch.from_numpy(widen(t)) for t in (q, k, v))
    zero = torch.zeros(B, H, 1, d, dtype=torch.float64)
    tk2, tv2 = torch.cat([zero, tk], 2), torch.cat([zero, tv], 2)
    idx = np.arange(L + 1)
    key_ok = idx[None, :] < (n[:, None] + 1)
    attn_mask = torch.from_numpy(np.ascontiguousarray(
        np.broadcast_to(key_ok[:, None, None, :], (B, 1, L, L + 1))))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk2, tv2, attn_mask=attn_mask)
    for b in range(B):
        np.testing.assert_allclose(o1[b, :, : n[b]], ref[b, :, : n[b]].numpy(), rtol=1e-10,
                                   atol=1e-13)
    # Same identity through the oracle itself: SOFTMAX over the extended keys.
    q2 = np.concatenate([np.zeros((B, H, 1, d), np.uint16), q], axis=2)
    k2 = np.concatenate([np.zeros((B, H, 1, d), np.uint16), k], axis=2)
    v2 = np.concatenate([np.zeros((B, H, 1, d), np.uint16), v], axis=2)
    o2, lse2 = oracle_lib.fwd(q2, k2, v2, n + 1, bias=BIAS_NONE, variant=SOFTMAX)
    # Row r of the original is row r + 1 of the extended problem.
    for b in range(B):
        np.testing.assert_allclose(o1[b, :, : n[b]], o2[b, :, 1 : n[b] + 1], rtol=1e-12,
                                   atol=1e-14)
        np.testing.assert_allclose(lse1[b, :, : n[b]], lse2[b, :, 1 : n[b] + 1], rtol=1e-12)


def test_row_sums_with_unit_values(oracle_lib):
    """V = 1: softmax rows sum to 1; softmax_1 rows to a value in (0, 1)."""
    rng = np.random.default_rng(7)
    B, H, L, d = 2, 2, 30, 4
    q, k, _ = random_inputs(rng, B, H, L, d)
    v = bf16(np.ones((B, H, L, d)))
    n = np.array([30, 11], np.int32)
    o, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX)
    o1, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX1)
    for b in range(B):
        np.testing.assert_allclose(o[b, :, : n[b]], 1.0, rtol=1e-13)
        s1 = o1[b, :, : n[b]]
        assert np.all(s1 > 0) and np.all(s1 < 1)


def test_softmax1_ratios_and_limits(oracle_lib):
    """softmax_1 keeps softmax's ratios; with very negative logits its terms
    tend to 0 while softmax's tend to 1/k (golden fixture)."""
    table = read_golden("softmax1_limits.txt")
    for k_val, lim_soft, lim_soft1 in table:
        kk = int(k_val)
        L = d = 16
        # Scores equal scale * q values (one-hot K, V); -8 * 16 * scale(=1) = -128.
        qv = np.full((L, d), -128.0)
        q, k, v = onehot_inputs(None, L, d, qv)
        n = np.array([kk], np.int32)
        o, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX, scale=1.0)
        o1, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX1, scale=1.0)
        np.testing.assert_allclose(o[0, 0, :kk, :kk], lim_soft, rtol=1e-14)
        assert np.all(np.abs(o1[0, 0, :kk, :kk] - lim_soft1) < 1e-50)
    rng = np.random.default_rng(8)
    L = d = 10
    q, k, v = onehot_inputs(rng, L, d, rng.standard_normal((L, d)) * 2)
    n = np.array([L], np.int32)
    p, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX, scale=1.0)
    p1, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX1, scale=1.0)
    ratio = p[0, 0, :, :L] / p[0, 0, :, :1]
    ratio1 = p1[0, 0, :, :L] / p1[0, 0, :, :1]
    np.testing.assert_allclose(ratio1, ratio, rtol=1e-12)
    s = widen(q[0, 0])[:, :L]
    np.testing.assert_allclose(ratio, np.exp(s - s[:, :1]), rtol=1e-12)
    assert np.all(p1[0, 0, :, :L].sum(axis=1) < 1)


def test_zero_queries_cross_variant(oracle_lib):
    """Q = 0: softmax_1 without bias and sigmoid with -ln n both give sum v / (1 + n)."""
    rng = np.random.default_rng(9)
    B, H, L, d = 3, 2, 21, 8
    _, k, v = random_inputs(rng, B, H, L, d)
    q = np.zeros_like(k)
    n = np.array([21, 5, 12], np.int32)
    a, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX1)
    b_, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_LOG_SEQLEN, variant=SIGMOID)
    np.testing.assert_allclose(a, b_, rtol=1e-13, atol=1e-15)
    s, _ = oracle_lib.fwd(q, k, v, n, bias=BIAS_NONE, variant=SOFTMAX)
    for bb in range(B):  # softmax of equal logits: the mean of the valid values
        want = widen(v[bb])[:, : n[bb]].mean(axis=1)
        np.testing.assert_allclose(s[bb, :, : n[bb]], np.broadcast_to(
            want[:, None, :], (H, n[bb], d)), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("variant", VARIANTS)
def test_key_permutation_invariance(oracle_lib, variant):
    rng = np.random.default_rng(10 + variant)
    B, H, L, d = 2, 2, 40, 8
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([37, 22], np.int32)
    mask = (rng.random((B, L, L)) < 0.7).astype(np.uint8)
    o, _ = oracle_lib.fwd(q, k, v, n, mask=mask, variant=variant)
    k2, v2, m2 = k.copy(), v.copy(), mask.copy()
    for b in range(B):
        perm = np.concatenate([rng.permutation(n[b]), np.arange(n[b], L)])
        k2[b] = k[b][:, perm]
        v2[b] = v[b][:, perm]
        m2[b] = mask[b][:, perm]
    o2, _ = oracle_lib.fwd(q, k2, v2, n, mask=m2, variant=variant)
    np.testing.assert_allclose(o2, o, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("bq,bk", [(32, 32), (16, 64), (64, 16)])
def test_block_skip_equals_dense(oracle_lib, variant, bq, bk):
    """Skipped tiles hold no valid element, so skipping changes nothing: the
    skip path equals the visit-all path bit for bit, and both equal the plain
    definition up to rounding order."""
    rng = np.random.default_rng(20 + variant + bq)
    B, H, L, d = 3, 2, 100, 8
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([100, 45, 0], np.int32)
    idx = np.arange(L)
    mask = np.zeros((B, L, L), np.uint8)
    for b in range(B):  # band + sparse pattern: many empty tiles
        band = np.abs(idx[:, None] - idx[None, :]) < 20
        mask[b] = (band | (rng.random((L, L)) < 0.002)).astype(np.uint8)
    bm = oracle_lib.blockmask(n, mask, L, bq, bk)
    assert 0 < bm.sum() < bm.size
    bias = BIAS_LOG_SEQLEN if variant == SIGMOID else BIAS_NONE
    skip, lse_s = oracle_lib.fwd_tiled(q, k, v, n, bm, bq, bk, mask=mask, bias=bias,
                                       variant=variant)
    full, lse_f = oracle_lib.fwd_tiled(q, k, v, n, None, bq, bk, mask=mask, bias=bias,
                                       variant=variant)
    dense, lse_d = oracle_lib.fwd(q, k, v, n, mask=mask, bias=bias, variant=variant)
    assert np.array_equal(skip, full) and np.array_equal(lse_s, lse_f)
    np.testing.assert_allclose(skip, dense, rtol=1e-11, atol=1e-14)
    if variant != SIGMOID:
        np.testing.assert_allclose(lse_s, lse_d, rtol=1e-12)


@pytest.mark.parametrize("variant", VARIANTS)
def test_padded_and_empty_rows_are_zero_and_poison_is_ignored(oracle_lib, variant):
    rng = np.random.default_rng(30 + variant)
    B, H, L, d = 2, 2, 50, 8
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([31, 50], np.int32)
    mask = (rng.random((B, L, L)) < 0.5).astype(np.uint8)
    mask[:, 3, :] = 0  # valid query row with no valid key
    o, lse = oracle_lib.fwd(q, k, v, n, mask=mask, variant=variant)
    qp, kp, vp = q.copy(), k.copy(), v.copy()
    nan = np.uint16(0x7FC0)
    for t in (qp, kp, vp):
        t[0, :, n[0]:] = nan
    op, lsep = oracle_lib.fwd(qp, kp, vp, n, mask=mask, variant=variant)
    assert np.array_equal(o, op) and np.array_equal(lse, lsep)
    assert np.all(o[0, :, n[0]:] == 0) and np.all(np.isneginf(lse[0, :, n[0]:]))
    assert np.all(o[:, :, 3] == 0)
    if variant == SOFTMAX1:  # log(1 + empty sum) = 0
        assert np.all(lse[:, :, 3] == 0)
    else:
        assert np.all(np.isneginf(lse[:, :, 3]))


@pytest.mark.parametrize("variant", VARIANTS)
def test_fp32_statement_agrees_with_fp64(oracle_lib, variant):
    rng = np.random.default_rng(40 + variant)
    B, H, L, d = 2, 2, 300, 64
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([300, 123], np.int32)
    bias = BIAS_LOG_SEQLEN if variant == SIGMOID else BIAS_NONE
    o64, _ = oracle_lib.fwd(q, k, v, n, bias=bias, variant=variant, precision="f64")
    o32, _ = oracle_lib.fwd(q, k, v, n, bias=bias, variant=variant, precision="f32")
    rel = np.linalg.norm(o32 - o64) / np.linalg.norm(o64)
    assert rel < 1e-5


def test_rows_api_matches_full(oracle_lib):
    rng = np.random.default_rng(50)
    B, H, L, d = 2, 2, 40, 8
    q, k, v = random_inputs(rng, B, H, L, d)
    n = np.array([40, 19], np.int32)
    for variant in VARIANTS:
        o, lse = oracle_lib.fwd(q, k, v, n, variant=variant)
        rows = [0, 5, 18, 19, 39]
        orows, lrows = oracle_lib.fwd_rows(q, k, v, n, 1, 1, rows, variant=variant)
        assert np.array_equal(orows, o[1, 1, rows]) and np.array_equal(lrows, lse[1, 1, rows])
