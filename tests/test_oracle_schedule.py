"""Pins of oracle.schedule (the work schedule written out from its
definition; Binary Block Masking, "Presentation" and "How it works"):
a hand-worked example, the invariants every schedule must meet (each tile
exactly once, its pair's XCD, longest sequence first; zero items after the
compute items of one kind when not more numerous, else spread between them,
and spread evenly over the second half of two kinds),
and the kept-entry lists against a vectorised numpy reduction of the block
mask (a different computation from the oracle's loops)."""
import numpy as np
import pytest

import oracle


def test_hand_worked_example():
    # Two sequences (n = 100, 300), one head, L = 300: the longer is rank 0
    # (pair 0 -> XCD 0: tiles 0, 1, 2 in slots 0, 8, 16), the shorter rank 1
    # (pair 1 -> XCD 1: tile 0 in slot 1, then one zero item for its fully
    # padded tiles 1 and 2 in slot 9).  24 slots = 8 XCDs x 1 pair x 3 tiles.
    bm = oracle.blockmask(np.array([100, 300], np.int32), None, 300, 128, 128)
    s = oracle.schedule([100, 300], bm, 1, 300, 128, 128)
    assert len(s["items1"]) == 24 and len(s["items2"]) == 48
    assert {i: x for i, x in enumerate(s["items1"]) if x} == {
        0: (1, 0, 0, 0, 300), 8: (1, 0, 0, 1, 300), 16: (1, 0, 0, 2, 300), 1: (0, 0, 0, 0, 100),
        9: (0, 0, 0, 1, 100)}
    # Two kinds: the pair's kind-0 tiles, then its kind-1 tiles.  XCD 1 has
    # two compute items and two zero items (kind 0, then kind 1): h = 1,
    # R = 1, so both follow compute item 1 + floor(j * 1 / 2) = 1.
    assert [x for x in s["items2"][0::8] if x] == [(1, 0, k, t, 300) for k in (0, 1) for t in range(3)]
    assert [x for x in s["items2"][1::8] if x] == [(0, 0, 0, 0, 100), (0, 0, 1, 0, 100),
                                                    (0, 0, 0, 1, 100), (0, 0, 1, 1, 100)]
    # n = 600 at L = 1200: tiles 0..4 hold valid rows, tiles 5..8 and 9 form
    # two zero items.  One kind: five compute items, two zero items (not more
    # numerous): compute items, then zero items.  Two kinds: ten compute
    # items (h = 5, R = 5) and four zero items, after compute items
    # 5 + floor(j * 5 / 4) = 5, 6, 7, 8.
    s5 = oracle.schedule([600], oracle.blockmask(np.array([600], np.int32), None, 1200, 128, 128),
                         1, 1200, 128, 128)
    assert [x[3] for x in s5["items1"] if x] == [0, 1, 2, 3, 4, 5, 9]
    # n = 200 at L = 2000: compute tiles 0, 1 and zero items at tiles 2, 6,
    # 10, 14 (more numerous): spread, zero item j after compute item
    # floor(j * 2 / 4) = 0, 0, 1, 1.
    s6 = oracle.schedule([200], oracle.blockmask(np.array([200], np.int32), None, 2000, 128, 128),
                         1, 2000, 128, 128)
    assert [x[3] for x in s6["items1"] if x] == [0, 2, 6, 1, 10, 14]
    assert [(x[2], x[3]) for x in s5["items2"] if x] == (
        [(0, t) for t in range(5)] + [(1, 0), (0, 5), (1, 1), (0, 9), (1, 2), (1, 5), (1, 3),
                                      (1, 9), (1, 4)])
    # An empty sequence among 9 tiles (L = 1100): zero items at tiles 0, 4, 8.
    s0 = oracle.schedule([0], oracle.blockmask(np.array([0], np.int32), None, 1100, 128, 128),
                         1, 1100, 128, 128)
    assert [x for x in s0["items1"] if x] == [(0, 0, 0, t, 0) for t in (0, 4, 8)]
    # Sequence 0 keeps only block (0, 0) (100 < 128); sequence 1 keeps all of
    # its 3 x 3 blocks, full where the block lies inside [0, 256)^2.
    assert s["qlists"][0] == [[(0, 1, 0)], [], []]
    assert s["qlists"][1] == [[(0, 1, 1), (1, 1, 1), (2, 1, 0)]] * 2 + [[(0, 1, 0), (1, 1, 0), (2, 1, 0)]]
    assert s["klists"] == s["qlists"]  # a symmetric block mask


def test_lines_of_a_group_and_their_bits():
    # block_q = 32: a 128-row group spans block rows 0..3; an entry kept by
    # rows 1 and 3 only carries kept bits 0b1010.
    L, n = 128, np.array([128], np.int32)
    bm = np.zeros((1, 4, 2), np.uint8)  # block_q 32, block_k 64
    bm[0, 1, 1] = 1
    bm[0, 3, 1] = 3
    bm[0, 0, 0] = 1
    s = oracle.schedule(n, bm, 1, L, 32, 64)
    assert s["qlists"][0] == [[(0, 0b0001, 0), (1, 0b1010, 0b1000)]]
    # Key group 0 spans block columns 0 and 1 (C = 2), entries down the 4 rows.
    assert s["klists"][0] == [[(0, 0b01, 0), (1, 0b10, 0), (3, 0b10, 0b10)]]


@pytest.mark.parametrize("seed", range(6))
def test_schedule_invariants(seed):
    rng = np.random.default_rng(seed)
    B, H = int(rng.integers(1, 20)), int(rng.integers(1, 11))
    L = int(rng.integers(1, 700))
    n = rng.integers(-5, L + 5, size=B).astype(np.int32)
    n[rng.integers(B)] = 0
    bq, bk = (32, 64, 128)[seed % 3], (128, 32, 64)[seed % 3]
    bm = oracle.blockmask(n, None, L, bq, bk)
    s = oracle.schedule(n, bm, H, L, bq, bk)
    nc = np.clip(n, 0, L)
    G = -(-L // 128)
    order = sorted(range(B), key=lambda b: (-nc[b], b))
    pair_of = {(order[r], h): r * H + h for r in range(B) for h in range(H)}
    for K, name in ((1, "items1"), (2, "items2")):
        slots = s[name]
        assert len(slots) == 8 * (-(-(B * H) // 8)) * G * K
        seen = [x for x in slots if x is not None]
        # A compute item covers its tile; a zero item (its tile at or past
        # ceil(n / 128)) covers ZERO_TILES tiles from there, below G.
        covered = []
        for b, h, kind, t, nb in seen:
            real = -(-nb // 128)
            if t < real:
                covered.append((b, h, kind, t))
            else:
                assert (t - real) % oracle.ZERO_TILES == 0  # runs start at the first padded tile
                covered += [(b, h, kind, u) for u in range(t, min(G, t + oracle.ZERO_TILES))]
            assert nb == nc[b]
        want = sorted((b, h, kind, t) for b in range(B) for h in range(H)
                      for kind in range(K) for t in range(G))
        assert sorted(covered) == want  # every tile exactly once
        for x in range(8):
            mine = [it for it in slots[x::8]]
            live = [it for it in mine if it is not None]
            assert mine[:len(live)] == live  # no hole before the last item
            for b, h, kind, t, nb in live:
                assert pair_of[(b, h)] % 8 == x  # the pair's XCD
            work = [t * 128 < nb for b, h, kind, t, nb in live]
            lens = [nb for (b, h, kind, t, nb), w in zip(live, work) if w]
            assert lens == sorted(lens, reverse=True)  # longest first
            # Zero items after the compute items (one kind), or spread evenly
            # over their second half (two kinds): none before compute item
            # h = floor(Nc / 2), and after each later one at most
            # ceil(Nz / (Nc - h)).
            n_c, n_z = sum(work), len(work) - sum(work)
            if n_c and n_z:
                runs = "".join("c" if w else "z" for w in work).split("c")[1:]
                if K == 1 and n_z <= n_c:
                    assert work == [True] * n_c + [False] * n_z
                elif K == 1:
                    assert work[0] and max(len(r) for r in runs) <= -(-n_z // n_c)
                else:
                    half = n_c // 2
                    assert all(len(r) == 0 for r in runs[:half])
                    assert max(len(r) for r in runs[half:]) <= -(-n_z // (n_c - half))


@pytest.mark.parametrize("bq,bk", [(32, 128), (64, 64), (128, 32)])
def test_lists_against_numpy_reduction(bq, bk):
    rng = np.random.default_rng(bq + bk)
    B, L = 3, 517
    n = np.array([517, 300, 0], np.int32)
    mask = (rng.random((B, L, L)) < 0.002).astype(np.uint8)
    mask[1, 100:260, 40:300] = 1
    bm = oracle.blockmask(n, mask, L, bq, bk)
    s = oracle.schedule(n, bm, 2, L, bq, bk)
    G, Tq, Tk = -(-L // 128), -(-L // bq), -(-L // bk)
    R, C = 128 // bq, 128 // bk
    for b in range(B):
        for g in range(G):
            rows = bm[b, g * R:min(g * R + R, Tq), :min(Tk, -(-int(n[b]) // bk))]  # [lines, e]
            w = (1 << np.arange(rows.shape[0]))[:, None]
            on, full = ((rows != 0) * w).sum(0), (((rows >> 1) & 1) * w).sum(0)
            want = [(int(e), int(on[e]), int(full[e])) for e in np.nonzero(on)[0]]
            assert s["qlists"][b][g] == want
            cols = bm[b, :min(Tq, -(-int(n[b]) // bq)), g * C:min(g * C + C, Tk)].T  # [lines, e]
            w = (1 << np.arange(cols.shape[0]))[:, None]
            on, full = ((cols != 0) * w).sum(0), (((cols >> 1) & 1) * w).sum(0)
            want = [(int(e), int(on[e]), int(full[e])) for e in np.nonzero(on)[0]]
            assert s["klists"][b][g] == want
