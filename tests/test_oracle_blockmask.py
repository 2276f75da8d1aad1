"""Pins for the oracle's binary block mask (Binary Block Masking page,
"Presentation": a block is kept when it holds at least one active entry; one
matrix per batch entry shared by all heads)."""
import numpy as np
import pytest

from synthetic import long_packed_docs, tiny_sigmoid


def closed_form_padding(seq_lens, L, bq, bk):
    """With padding only, block (i, j) is non-empty iff both tiles start below n."""
    n = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, L)
    Tq, Tk = -(-L // bq), -(-L // bk)
    i = np.arange(Tq)[None, :, None]
    j = np.arange(Tk)[None, None, :]
    nb = n[:, None, None]
    return ((i * bq < nb) & (j * bk < nb)).astype(np.uint8)


def blockwise_any(valid, bq, bk):
    """Pad the element validity to whole tiles and OR-reduce each tile with numpy."""
    B, L, _ = valid.shape
    Tq, Tk = -(-L // bq), -(-L // bk)
    padded = np.zeros((B, Tq * bq, Tk * bk), dtype=bool)
    padded[:, :L, :L] = valid
    return padded.reshape(B, Tq, bq, Tk, bk).any(axis=(2, 4)).astype(np.uint8)


@pytest.mark.parametrize("L,bq,bk", [(128, 32, 32), (100, 32, 32), (257, 64, 128),
                                     (129, 128, 64), (5, 32, 32), (1, 32, 128)])
def test_padding_only_matches_closed_form(oracle_lib, L, bq, bk):
    rng = np.random.default_rng(L * 7 + bq)
    n = rng.integers(-3, L + 4, size=9).astype(np.int32)
    n[:4] = [0, L, 1, min(L, bq)]
    got = oracle_lib.blockmask(n, None, L, bq, bk)
    np.testing.assert_array_equal(got, closed_form_padding(n, L, bq, bk))


@pytest.mark.parametrize("L,bq,bk,density", [(96, 32, 32, 0.02), (130, 64, 32, 0.001),
                                             (77, 32, 64, 0.3), (200, 128, 128, 0.0005)])
def test_arbitrary_mask_matches_blockwise_any(oracle_lib, L, bq, bk, density):
    rng = np.random.default_rng(L + bk)
    B = 3
    n = np.array([L, L // 2 + 1, 0], dtype=np.int32)
    mask = (rng.random((B, L, L)) < density).astype(np.uint8)
    got = oracle_lib.blockmask(n, mask, L, bq, bk)
    idx = np.arange(L)
    inside = (idx[None, :, None] < n[:, None, None]) & (idx[None, None, :] < n[:, None, None])
    want = blockwise_any(inside & (mask != 0), bq, bk)
    np.testing.assert_array_equal(got, want)
    assert got[2].sum() == 0  # n = 0: nothing valid


def test_values_are_zero_or_one(oracle_lib):
    w = long_packed_docs(tensors=())
    bm = oracle_lib.blockmask(w.seq_lens, w.mask, w.L, 128, 128)
    assert set(np.unique(bm).tolist()) <= {0, 1}
    # Same result as the numpy tile reduction on this structured mask.
    idx = np.arange(w.L)
    n = np.clip(w.seq_lens, 0, w.L)
    inside = (idx[None, :, None] < n[:, None, None]) & (idx[None, None, :] < n[:, None, None])
    np.testing.assert_array_equal(bm, blockwise_any(inside & (w.mask != 0), 128, 128))
    # Causal packed documents: no block strictly above the diagonal survives.
    Tq = bm.shape[1]
    assert all(bm[:, i, j].sum() == 0 for i in range(Tq) for j in range(i + 1, Tq))


def test_tiny_workload_block_count(oracle_lib):
    w = tiny_sigmoid(tensors=())
    bm = oracle_lib.blockmask(w.seq_lens, None, w.L, 32, 32)
    tiles = np.ceil(w.seq_lens / 32).astype(int)
    assert bm.sum() == int((tiles ** 2).sum())


@pytest.mark.parametrize("L,bq,bk", [(96, 32, 32), (100, 64, 32), (130, 32, 128)])
def test_single_element_at_tile_edges(oracle_lib, L, bq, bk):
    """One active element per mask, placed on the first and last row and column
    of tiles (and in the clipped last tile): exactly its own block is set."""
    edges_r = sorted({0, bq - 1, bq, L - 1, (L - 1) // bq * bq})
    edges_c = sorted({0, bk - 1, bk, L - 1, (L - 1) // bk * bk})
    for r in edges_r:
        for c in edges_c:
            mask = np.zeros((1, L, L), np.uint8)
            mask[0, r, c] = 1
            bm = oracle_lib.blockmask(np.array([L], np.int32), mask, L, bq, bk)
            want = np.zeros_like(bm)
            want[0, r // bq, c // bk] = 1
            np.testing.assert_array_equal(bm, want, err_msg=f"element ({r}, {c})")
