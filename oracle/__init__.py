"""CPU oracle for padded variable-length attention.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may use this package; the GPU library never
does.  It wraps ``oracle.c`` (plain C, compiled with gcc) through ctypes and
drives it one (batch entry, head) slice at a time on a thread pool (ctypes
releases the GIL during each call).

All tensors are numpy ``uint16`` arrays of bf16 bit patterns laid out
``[B, H, L, d]``; results are float64 (``precision="f64"``) or float32
(``precision="f32"``).  Every function cites the passage it follows in
``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SIGMOID, SOFTMAX, SOFTMAX1 = 0, 1, 2
BIAS_NONE, BIAS_LOG_SEQLEN, BIAS_LOG_PADLEN = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c twice (double and float) into liboracle.so with gcc."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    flags = ["-O2", "-std=c11", "-fPIC", "-fno-fast-math", "-Wall", "-Wextra"]
    objs = []
    for real, sfx, extra in (("double", "_f64", ["-DORACLE_WITH_BLOCKMASK"]),
                             ("float", "_f32", [])):
        obj = os.path.join(_HERE, f"oracle{sfx}.o")
        subprocess.check_call(["gcc", *flags, f"-DREAL={real}", f"-DSFX={sfx}", *extra,
                               "-c", _SRC, "-o", obj])
        objs.append(obj)
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-shared", "-o", tmp, *objs, "-lm"])
    os.replace(tmp, _LIB_PATH)
    for obj in objs:
        os.remove(obj)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    for sfx, R in (("_f64", ctypes.c_double), ("_f32", ctypes.c_float)):
        f = getattr(lib, "oracle_fwd_rows" + sfx)
        f.argtypes = [I, I, I, P, P, P, P, I, I, R, I, I, P, P]
        f.restype = None
        f = getattr(lib, "oracle_fwd_tiled" + sfx)
        f.argtypes = [I, I, I, P, P, P, P, P, I, I, I, I, R, P, P]
        f.restype = None
        f = getattr(lib, "oracle_bwd_dq_rows" + sfx)
        f.argtypes = [I, I, I, P, P, P, P, P, P, I, I, R, I, I, P]
        f.restype = None
        f = getattr(lib, "oracle_bwd_dkv_rows" + sfx)
        f.argtypes = [I, I, I, P, P, P, P, P, P, I, I, R, I, I, P, P]
        f.restype = None
    lib.oracle_blockmask.argtypes = [P, P, I, I, I, I, P]
    lib.oracle_blockmask.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype(precision):
    return {"f64": np.float64, "f32": np.float32}[precision]


def _threads(threads):
    """Worker threads: as asked, else every CPU the process sees, capped by
    OMP_NUM_THREADS when it is set (a machine's share of cores per GPU)."""
    if threads:
        return threads
    n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(cap)) if cap.isdigit() and int(cap) > 0 else n


def default_scale(d: int) -> float:
    """1/sqrt(d), d the head dimension (the scaled dot product of both pages)."""
    return 1.0 / float(np.sqrt(d))


def key_range_mask(key_range, L: int) -> np.ndarray:
    """The element mask that key ranges stand for: uint8 [B, L, L] with
    mask[b, r, c] = 1 iff key_range[b, r, 0] <= c <= key_range[b, r, 1]
    (the definition in include/sigattn.h, written out)."""
    kr = np.asarray(key_range, dtype=np.int64)
    c = np.arange(L)[None, None, :]
    return ((kr[:, :, 0:1] <= c) & (c <= kr[:, :, 1:2])).astype(np.uint8)


def _element_mask(mask, key_range, L):
    """The dense element mask of a call: ``mask`` itself, or the one the key
    ranges stand for.  A call takes one form or the other (as the C ABI)."""
    if key_range is None:
        return mask
    if mask is not None:
        raise ValueError("mask and key_range are alternative forms of one element mask")
    return key_range_mask(key_range, L)


def blockmask(seq_lens, mask, L: int, block_q: int, block_k: int, key_range=None) -> np.ndarray:
    """Block matrix [B, Tq, Tk] (uint8): bit 0 the binary block mask (tile holds
    a valid element), bit 1 a full tile (inside [0, n)^2, every element valid);
    see oracle_blockmask.  ``key_range`` [B, L, 2] stands for key_range_mask."""
    mask = _element_mask(mask, key_range, L)
    lib = _load()
    n = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = n.shape[0]
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    Tq, Tk = -(-L // block_q), -(-L // block_k)
    out = np.zeros((B, Tq, Tk), dtype=np.uint8)
    lib.oracle_blockmask(_ptr(n), _ptr(m), B, L, block_q, block_k, _ptr(out))
    return out


def _heads(q):
    B, H, L, d = q.shape
    return B, H, L, d


def fwd(q, k, v, seq_lens, mask=None, bias=BIAS_LOG_SEQLEN, variant=SIGMOID, scale=None,
        precision="f64", threads=None, heads=None, key_range=None):
    """Forward by the plain definition (oracle_fwd_rows) for every row.

    Returns (o [B, H, L, d], lse [B, H, L]).  ``heads``: optional list of
    (b, h) pairs to compute; the others are left at zero / -inf.
    """
    mask = _element_mask(mask, key_range, q.shape[2])
    lib = _load()
    B, H, L, d = _heads(q)
    dt = _dtype(precision)
    fn = getattr(lib, "oracle_fwd_rows_" + precision)
    scale = default_scale(d) if scale is None else scale
    o = np.zeros((B, H, L, d), dtype=dt)
    lse = np.full((B, H, L), -np.inf, dtype=dt)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        qs, ks, vs = (np.ascontiguousarray(t[b, h]) for t in (q, k, v))
        mb = None if mask is None else np.ascontiguousarray(mask[b])
        ob = np.zeros((L, d), dtype=dt)
        lb = np.zeros(L, dtype=dt)
        fn(L, d, int(seq_lens[b]), _ptr(qs), _ptr(ks), _ptr(vs), _ptr(mb), bias, variant,
           scale, 0, L, _ptr(ob), _ptr(lb))
        o[b, h] = ob
        lse[b, h] = lb

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(one, pairs))
    return o, lse


def fwd_rows(q, k, v, seq_lens, b: int, h: int, rows, mask=None, bias=BIAS_LOG_SEQLEN,
             variant=SIGMOID, scale=None, precision="f64", key_range=None):
    """Selected output rows of one head: (o [len(rows), d], lse [len(rows)])."""
    lib = _load()
    B, H, L, d = _heads(q)
    dt = _dtype(precision)
    fn = getattr(lib, "oracle_fwd_rows_" + precision)
    scale = default_scale(d) if scale is None else scale
    qs, ks, vs = (np.ascontiguousarray(t[b, h]) for t in (q, k, v))
    # Only batch entry b's mask is needed (its key ranges written out).
    mb = None if mask is None else np.ascontiguousarray(mask[b])
    if key_range is not None:
        mb = _element_mask(None if mb is None else mb[None], key_range[b:b + 1], L)[0]
    rows = list(rows)
    o = np.zeros((len(rows), d), dtype=dt)
    lse = np.zeros(len(rows), dtype=dt)
    one_o = np.zeros((1, d), dtype=dt)
    one_l = np.zeros(1, dtype=dt)
    for i, r in enumerate(rows):
        fn(L, d, int(seq_lens[b]), _ptr(qs), _ptr(ks), _ptr(vs), _ptr(mb), bias, variant,
           scale, int(r), int(r) + 1, _ptr(one_o), _ptr(one_l))
        o[i] = one_o[0]
        lse[i] = one_l[0]
    return o, lse


def fwd_tiled(q, k, v, seq_lens, block_mask=None, block_q=64, block_k=64, mask=None,
              bias=BIAS_LOG_SEQLEN, variant=SIGMOID, scale=None, precision="f64",
              threads=None, key_range=None):
    """Forward by the tiled online algorithm (oracle_fwd_tiled).

    ``block_mask`` [B, Tq, Tk] selects the tiles visited; None visits all.
    """
    mask = _element_mask(mask, key_range, q.shape[2])
    lib = _load()
    B, H, L, d = _heads(q)
    dt = _dtype(precision)
    fn = getattr(lib, "oracle_fwd_tiled_" + precision)
    scale = default_scale(d) if scale is None else scale
    o = np.zeros((B, H, L, d), dtype=dt)
    lse = np.zeros((B, H, L), dtype=dt)

    def one(bh):
        b, h = bh
        qs, ks, vs = (np.ascontiguousarray(t[b, h]) for t in (q, k, v))
        mb = None if mask is None else np.ascontiguousarray(mask[b])
        bmb = None if block_mask is None else np.ascontiguousarray(block_mask[b], dtype=np.uint8)
        ob = np.zeros((L, d), dtype=dt)
        lb = np.zeros(L, dtype=dt)
        fn(L, d, int(seq_lens[b]), _ptr(qs), _ptr(ks), _ptr(vs), _ptr(mb), _ptr(bmb),
           block_q, block_k, bias, variant, scale, _ptr(ob), _ptr(lb))
        o[b, h] = ob
        lse[b, h] = lb

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(one, [(b, h) for b in range(B) for h in range(H)]))
    return o, lse


def bwd(q, k, v, do, seq_lens, mask=None, bias=BIAS_LOG_SEQLEN, variant=SIGMOID, scale=None,
        precision="f64", threads=None, heads=None, key_range=None, o=None):
    """dQ, dK, dV [B, H, L, d] by the plain definition (oracle_bwd_*_rows).

    ``o``: the forward output the backward is handed (bf16 bits [B, H, L, d],
    softmax family only), from which D = rowsum(dO * O) is formed, as the
    library's backward forms it from the O it is given; None for the exact
    output."""
    mask = _element_mask(mask, key_range, q.shape[2])
    lib = _load()
    B, H, L, d = _heads(q)
    dt = _dtype(precision)
    fq = getattr(lib, "oracle_bwd_dq_rows_" + precision)
    fkv = getattr(lib, "oracle_bwd_dkv_rows_" + precision)
    scale = default_scale(d) if scale is None else scale
    dq = np.zeros((B, H, L, d), dtype=dt)
    dk = np.zeros((B, H, L, d), dtype=dt)
    dv = np.zeros((B, H, L, d), dtype=dt)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]

    def one(bh):
        b, h = bh
        qs, ks, vs, ds = (np.ascontiguousarray(t[b, h]) for t in (q, k, v, do))
        os_ = None if o is None else np.ascontiguousarray(o[b, h])
        mb = None if mask is None else np.ascontiguousarray(mask[b])
        gq = np.zeros((L, d), dtype=dt)
        gk = np.zeros((L, d), dtype=dt)
        gv = np.zeros((L, d), dtype=dt)
        n = int(seq_lens[b])
        fq(L, d, n, _ptr(qs), _ptr(ks), _ptr(vs), _ptr(ds), _ptr(os_), _ptr(mb), bias, variant,
           scale, 0, L, _ptr(gq))
        fkv(L, d, n, _ptr(qs), _ptr(ks), _ptr(vs), _ptr(ds), _ptr(os_), _ptr(mb), bias, variant,
            scale, 0, L, _ptr(gk), _ptr(gv))
        dq[b, h], dk[b, h], dv[b, h] = gq, gk, gv

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(one, pairs))
    return dq, dk, dv


def bwd_rows(q, k, v, do, seq_lens, b: int, h: int, q_rows, k_rows, mask=None,
             bias=BIAS_LOG_SEQLEN, variant=SIGMOID, scale=None, precision="f64", key_range=None,
             o=None):
    """Selected rows of one head: (dq [len(q_rows), d], dk, dv [len(k_rows), d]);
    ``o`` as for bwd."""
    lib = _load()
    B, H, L, d = _heads(q)
    dt = _dtype(precision)
    fq = getattr(lib, "oracle_bwd_dq_rows_" + precision)
    fkv = getattr(lib, "oracle_bwd_dkv_rows_" + precision)
    scale = default_scale(d) if scale is None else scale
    qs, ks, vs, ds = (np.ascontiguousarray(t[b, h]) for t in (q, k, v, do))
    os_ = None if o is None else np.ascontiguousarray(o[b, h])
    # Only batch entry b's mask is needed (its key ranges written out).
    mb = None if mask is None else np.ascontiguousarray(mask[b])
    if key_range is not None:
        mb = _element_mask(None if mb is None else mb[None], key_range[b:b + 1], L)[0]
    n = int(seq_lens[b])
    q_rows, k_rows = list(q_rows), list(k_rows)
    dq = np.zeros((len(q_rows), d), dtype=dt)
    for i, r in enumerate(q_rows):
        row = np.zeros((1, d), dtype=dt)
        fq(L, d, n, _ptr(qs), _ptr(ks), _ptr(vs), _ptr(ds), _ptr(os_), _ptr(mb), bias, variant,
           scale, int(r), int(r) + 1, _ptr(row))
        dq[i] = row[0]
    dk = np.zeros((len(k_rows), d), dtype=dt)
    dv = np.zeros((len(k_rows), d), dtype=dt)
    if k_rows:
        # One call per contiguous run keeps the softmax row statistics shared.
        lo, hi = min(k_rows), max(k_rows) + 1
        gk = np.zeros((hi - lo, d), dtype=dt)
        gv = np.zeros((hi - lo, d), dtype=dt)
        fkv(L, d, n, _ptr(qs), _ptr(ks), _ptr(vs), _ptr(ds), _ptr(os_), _ptr(mb), bias, variant,
            scale, lo, hi, _ptr(gk), _ptr(gv))
        for i, c in enumerate(k_rows):
            dk[i] = gk[c - lo]
            dv[i] = gv[c - lo]
    return dq, dk, dv


def diff_fwd(q1, k1, q2, k2, v, seq_lens, lam: float, mask=None, bias=BIAS_NONE, scale=None,
             precision="f64", threads=None, heads=None, key_range=None):
    """Differential attention ("Differential Transformer" note, "How
    differential attention works"): (softmax(S1) - lam softmax(S2)) V, each map
    the SOFTMAX of ``fwd`` over the same valid (r, c).  Returns
    (o, lse1, lse2)."""
    o1, lse1 = fwd(q1, k1, v, seq_lens, mask=mask, bias=bias, variant=SOFTMAX, scale=scale,
                   precision=precision, threads=threads, heads=heads, key_range=key_range)
    o2, lse2 = fwd(q2, k2, v, seq_lens, mask=mask, bias=bias, variant=SOFTMAX, scale=scale,
                   precision=precision, threads=threads, heads=heads, key_range=key_range)
    return o1 - lam * o2, lse1, lse2


def diff_fwd_rows(q1, k1, q2, k2, v, seq_lens, lam: float, b: int, h: int, rows, mask=None,
                  bias=BIAS_NONE, scale=None, precision="f64", key_range=None):
    """Selected output rows of one head of diff_fwd: o [len(rows), d]."""
    o1, _ = fwd_rows(q1, k1, v, seq_lens, b, h, rows, mask=mask, bias=bias, variant=SOFTMAX,
                     scale=scale, precision=precision, key_range=key_range)
    o2, _ = fwd_rows(q2, k2, v, seq_lens, b, h, rows, mask=mask, bias=bias, variant=SOFTMAX,
                     scale=scale, precision=precision, key_range=key_range)
    return o1 - lam * o2


def diff_bwd(q1, k1, q2, k2, v, do, seq_lens, lam: float, mask=None, bias=BIAS_NONE, scale=None,
             precision="f64", threads=None, key_range=None, o1=None, o2=None):
    """Gradients (dq1, dk1, dq2, dk2, dv) of sum(do * o), o = diff_fwd(...).
    The output is o1 - lam o2, linear in the two maps: map 1's gradients are
    the SOFTMAX backward with do, map 2's are -lam times it, dv adds both.
    o1, o2: each map's output as the backward is handed it (see bwd)."""
    g1 = bwd(q1, k1, v, do, seq_lens, mask=mask, bias=bias, variant=SOFTMAX, scale=scale,
             precision=precision, threads=threads, key_range=key_range, o=o1)
    g2 = bwd(q2, k2, v, do, seq_lens, mask=mask, bias=bias, variant=SOFTMAX, scale=scale,
             precision=precision, threads=threads, key_range=key_range, o=o2)
    return g1[0], g1[1], -lam * g2[0], -lam * g2[1], g1[2] - lam * g2[2]


def diff_bwd_rows(q1, k1, q2, k2, v, do, seq_lens, lam: float, b: int, h: int, q_rows, k_rows,
                  mask=None, bias=BIAS_NONE, scale=None, precision="f64", key_range=None):
    """Selected rows of one head of diff_bwd: (dq1 [len(q_rows), d], dk1
    [len(k_rows), d], dq2, dk2, dv), by the same linearity (each map's SOFTMAX
    backward rows with do; map 2's scaled by -lam; dv the sum)."""
    kw = dict(mask=mask, bias=bias, variant=SOFTMAX, scale=scale, precision=precision,
              key_range=key_range)
    dq1, dk1, dv1 = bwd_rows(q1, k1, v, do, seq_lens, b, h, q_rows, k_rows, **kw)
    dq2, dk2, dv2 = bwd_rows(q2, k2, v, do, seq_lens, b, h, q_rows, k_rows, **kw)
    return dq1, dk1, -lam * dq2, -lam * dk2, dv1 - lam * dv2


# Fully padded 128-row tiles per zero item of a work schedule.
ZERO_TILES = 4


def schedule(seq_lens, block_mask, H: int, L: int, block_q: int, block_k: int) -> dict:
    """Work schedule of one batch, by its definition (Binary Block Masking,
    "Presentation": the block structure is built once and shared by every
    head; "How it works": only the kept blocks are visited), written out with
    plain loops.

    Work items cover 128-row tiles of every (batch entry, head).  The pairs
    are ordered by length rank (longest first, ties by index; batches of more
    than 1024 entries keep index order) and then head; pair p goes to XCD
    p % 8.  XCD x lists, for its pairs in order, the ceil(n/128) tiles with
    valid rows (all tiles of kind 0, then of kind 1 when there are two
    kinds): the compute items; and, for its pairs again, zero items: the
    fully padded tiles ceil(n/128) .. ceil(L/128) - 1 (every tile of an
    empty sequence) in runs of ZERO_TILES, one item per run, named by its
    first tile (kind 0 runs, then kind 1).  With Nc compute and Nz zero
    items, h = Nc when there is one kind and Nz <= Nc, h = 0 when there is
    one kind and Nz > Nc, h = floor(Nc / 2) with two kinds; with R = Nc - h,
    zero item j follows compute item h + floor(j R / Nz), and when R = 0 all
    zero items follow the compute items.  Its k-th item sits in slot
    8 k + x; slots past the end are None.  Items are (b, h, kind, tile, n)
    with n = clamp(seq_lens[b]).

    Kept-entry lists: for batch entry b and 128-row query group g, the lines
    are the block rows g R .. g R + R - 1 (R = 128 / block_q) below Tq, and the
    entries e < min(Tk, ceil(n / block_k)) that some line keeps, increasing,
    each with the bits of the lines that keep it and of those whose entry is
    3 (full).  Key groups the same down the block columns (C = 128 / block_k,
    entries e < min(Tq, ceil(n / block_q))).

    Returns {"items1": [...], "items2": [...], "qlists": [[...] per g] per b,
    "klists": likewise}."""
    n = [int(min(max(int(x), 0), L)) for x in seq_lens]
    B = len(n)
    bm = np.asarray(block_mask)
    G = -(-L // 128)
    Tq, Tk = -(-L // block_q), -(-L // block_k)
    order = sorted(range(B), key=lambda b: (-n[b], b)) if B <= 1024 else list(range(B))
    pairs = [(order[r], h) for r in range(B) for h in range(H)]
    per_xcd = -(-(B * H) // 8)
    out = {}
    for K, name in ((1, "items1"), (2, "items2")):
        slots = [None] * (8 * per_xcd * G * K)
        for x in range(8):
            compute, zero = [], []
            for p in range(x, B * H, 8):
                b, h = pairs[p]
                if n[b] > 0:
                    compute += [(b, h, kind, t, n[b]) for kind in range(K)
                                for t in range(-(-n[b] // 128))]
            for p in range(x, B * H, 8):
                b, h = pairs[p]
                real = -(-n[b] // 128)
                zero += [(b, h, kind, t, n[b]) for kind in range(K)
                         for t in range(real, G, ZERO_TILES)]
            if K == 2:
                first = len(compute) // 2
            else:
                first = len(compute) if len(zero) <= len(compute) else 0
            rest = len(compute) - first
            if rest == 0:
                seq = compute + zero
            else:
                seq = []
                for c, item in enumerate(compute):
                    seq.append(item)
                    seq += [z for j, z in enumerate(zero) if first + j * rest // len(zero) == c]
            for k, item in enumerate(seq):
                slots[8 * k + x] = item
        out[name] = slots

    def entries(b, lines, nblk, value):
        kept = []
        for e in range(nblk):
            on = sum(1 << r for r, ln in enumerate(lines) if value(b, ln, e) != 0)
            full = sum(1 << r for r, ln in enumerate(lines) if value(b, ln, e) & 2)
            if on:
                kept.append((e, on, full))
        return kept

    R, C = 128 // block_q, 128 // block_k
    out["qlists"] = [[entries(b, [g * R + r for r in range(R) if g * R + r < Tq],
                              min(Tk, -(-n[b] // block_k)), lambda b_, ln, e: int(bm[b_, ln, e]))
                      for g in range(G)] for b in range(B)]
    out["klists"] = [[entries(b, [g * C + c for c in range(C) if g * C + c < Tk],
                              min(Tq, -(-n[b] // block_q)), lambda b_, ln, e: int(bm[b_, e, ln]))
                      for g in range(G)] for b in range(B)]
    return out
