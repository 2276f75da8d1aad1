"""Pins for the oracle's binary block mask (Binary Block Masking page,
"Presentation": a block is kept when it holds at least one active entry; one
matrix per batch entry shared by all heads).  Bit 0 of an entry is that binary
matrix; bit 1 marks full tiles (inside [0, n)^2 with every element valid)."""
import numpy as np
import pytest

from synthetic import long_packed_docs, tiny_sigmoid


def closed_form_padding(seq_lens, L, bq, bk):
    """With padding only, block (i, j) is non-empty iff both tiles start below
    n, and full iff both tiles end at or below n."""
    n = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, L)
    Tq, Tk = -(-L // bq), -(-L // bk)
    i = np.arange(Tq)[None, :, None]
    j = np.arange(Tk)[None, None, :]
    nb = n[:, None, None]
    any_ = (i * bq < nb) & (j * bk < nb)
    full = ((i + 1) * bq <= nb) & ((j + 1) * bk <= nb)
    return (any_ | (full << 1)).astype(np.uint8)


def blockwise_any(valid, bq, bk):
    """Pad the element validity to whole tiles and OR-reduce each tile with numpy."""
    B, L, _ = valid.shape
    Tq, Tk = -(-L // bq), -(-L // bk)
    padded = np.zeros((B, Tq * bq, Tk * bk), dtype=bool)
    padded[:, :L, :L] = valid
    return padded.reshape(B, Tq, bq, Tk, bk).any(axis=(2, 4)).astype(np.uint8)


def blockwise_full(valid, bq, bk):
    """Pad with invalid entries to whole tiles and AND-reduce each tile: a tile
    cut by L or holding any invalid element is not full."""
    B, L, _ = valid.shape
    Tq, Tk = -(-L // bq), -(-L // bk)
    padded = np.zeros((B, Tq * bq, Tk * bk), dtype=bool)
    padded[:, :L, :L] = valid
    return padded.reshape(B, Tq, bq, Tk, bk).all(axis=(2, 4)).astype(np.uint8)


def blockwise(valid, bq, bk):
    return blockwise_any(valid, bq, bk) | (blockwise_full(valid, bq, bk) << 1)


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
    want = blockwise(inside & (mask != 0), bq, bk)
    np.testing.assert_array_equal(got, want)
    assert got[2].sum() == 0  # n = 0: nothing valid


@pytest.mark.parametrize("L,bq,bk", [(96, 32, 32), (200, 64, 32), (257, 128, 64)])
def test_full_tiles_of_a_causal_mask(oracle_lib, L, bq, bk):
    """Lower-triangular mask: a tile is full exactly when it lies inside
    [0, n)^2 and its top-right corner (first row, last column) is valid."""
    n = np.array([L, L - 40, bq], np.int32)
    idx = np.arange(L)
    mask = np.broadcast_to((idx[None, :] <= idx[:, None]).astype(np.uint8), (3, L, L)).copy()
    got = oracle_lib.blockmask(n, mask, L, bq, bk)
    assert set(np.unique(got).tolist()) <= {0, 1, 3}
    for b in range(3):
        nb = int(n[b])
        for i in range(got.shape[1]):
            for j in range(got.shape[2]):
                inside = (i + 1) * bq <= nb and (j + 1) * bk <= nb
                corner = (j + 1) * bk - 1 <= i * bq
                any_ = i * bq < nb and j * bk < nb and j * bk <= min((i + 1) * bq, nb) - 1
                assert got[b, i, j] == (int(any_) | (int(inside and corner) << 1)), (b, i, j)


def test_values_are_zero_one_or_three(oracle_lib):
    w = long_packed_docs(tensors=())
    bm = oracle_lib.blockmask(w.seq_lens, w.mask, w.L, 128, 128)
    assert set(np.unique(bm).tolist()) <= {0, 1, 3}
    # Same result as the numpy tile reductions on this structured mask.
    idx = np.arange(w.L)
    n = np.clip(w.seq_lens, 0, w.L)
    inside = (idx[None, :, None] < n[:, None, None]) & (idx[None, None, :] < n[:, None, None])
    np.testing.assert_array_equal(bm, blockwise(inside & (w.mask != 0), 128, 128))
    assert (bm == 3).sum() > 0 and (bm == 1).sum() > 0
    # Causal packed documents: no block strictly above the diagonal survives.
    Tq = bm.shape[1]
    assert all(bm[:, i, j].sum() == 0 for i in range(Tq) for j in range(i + 1, Tq))


def test_tiny_workload_block_count(oracle_lib):
    w = tiny_sigmoid(tensors=())
    bm = oracle_lib.blockmask(w.seq_lens, None, w.L, 32, 32)
    tiles = np.ceil(w.seq_lens / 32).astype(int)
    assert (bm & 1).sum() == int((tiles ** 2).sum())
    whole = w.seq_lens // 32
    assert (bm >> 1).sum() == int((whole ** 2).sum())


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
