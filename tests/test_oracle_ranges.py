"""Pins for key-range element masks (one interval of keys per query row; the
packed-document masks that Binary Block Masking, "Applications and real-world
tests", counts among its targets).  The oracle turns ranges into the dense
mask they stand for; these tests check that conversion against independent
constructions and the block mask built from either form."""
import numpy as np
import pytest

import synthetic as syn


def test_causal_ranges_are_the_lower_triangle(oracle_lib):
    L = 37
    r = np.arange(L)
    kr = np.stack([np.zeros(L, np.int32), r.astype(np.int32)], axis=1)[None]
    np.testing.assert_array_equal(oracle_lib.key_range_mask(kr, L)[0],
                                  np.tril(np.ones((L, L), np.uint8)))


def test_empty_and_clipped_ranges(oracle_lib):
    L = 10
    kr = np.array([[[3, 2], [-5, 1], [8, 40], [0, -1], [4, 4]] + [[1, 0]] * 5], np.int32)
    m = oracle_lib.key_range_mask(kr, L)[0]
    assert m[0].sum() == 0 and m[3].sum() == 0          # lo > hi: nothing
    assert list(np.nonzero(m[1])[0]) == [0, 1]          # clipped below at 0
    assert list(np.nonzero(m[2])[0]) == [8, 9]          # clipped above at L - 1
    assert list(np.nonzero(m[4])[0]) == [4]


def test_packed_document_ranges_match_the_dense_mask(oracle_lib):
    w = syn.make_workload("docs", seed=3, B=3, H=1, d=8, lengths="uniform", lo=100, hi=700,
                          docs=True, tensors=())
    np.testing.assert_array_equal(oracle_lib.key_range_mask(w.key_range, w.L), w.mask)


@pytest.mark.parametrize("L,bq,bk", [(300, 64, 64), (257, 128, 32), (96, 32, 128)])
def test_block_mask_from_ranges_equals_dense(oracle_lib, L, bq, bk):
    """Sliding windows of random width, and rows past n: the block matrix from
    ranges is the one from the dense mask they stand for, which matches a
    brute-force tile reduction."""
    rng = np.random.default_rng(L + bq)
    B = 3
    n = np.array([L, L - 41, 5], np.int32)
    r = np.arange(L)
    width = rng.integers(0, 90, size=(B, L))
    kr = np.stack([r[None, :] - width, r[None, :] + rng.integers(-3, 4, size=(B, L))],
                  axis=2).astype(np.int32)
    dense = oracle_lib.key_range_mask(kr, L)
    got = oracle_lib.blockmask(n, None, L, bq, bk, key_range=kr)
    np.testing.assert_array_equal(got, oracle_lib.blockmask(n, dense, L, bq, bk))
    valid = dense.astype(bool) & (r[None, :, None] < n[:, None, None]) & (r[None, None, :] < n[:, None, None])
    Tq, Tk = -(-L // bq), -(-L // bk)
    pad = np.zeros((B, Tq * bq, Tk * bk), bool)
    pad[:, :L, :L] = valid
    tiles = pad.reshape(B, Tq, bq, Tk, bk)
    want = tiles.any(axis=(2, 4)).astype(np.uint8) | (tiles.all(axis=(2, 4)).astype(np.uint8) << 1)
    np.testing.assert_array_equal(got, want)


def test_one_element_mask_form_per_call():
    """Like the C ABI, the oracle takes a dense mask or key ranges, not both."""
    import oracle
    n = np.array([5], np.int32)
    with pytest.raises(ValueError):
        oracle.blockmask(n, np.ones((1, 8, 8), np.uint8), 8, 4, 4,
                         key_range=np.zeros((1, 8, 2), np.int32))
