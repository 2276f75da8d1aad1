"""Seeded synthetic workloads for padded variable-length attention.

This module only produces inputs: sequence lengths, packed-document masks and
bf16 tensors.  It holds none of the attention arithmetic, so both the GPU path
(tests, benchmark) and the CPU oracle can consume what it makes without
sharing any computation.

Recipes (all draws from one ``numpy.random.default_rng(seed)``, in this order:
lengths, then documents per batch entry, then Q, K, V, dO):

* lengths ``uniform``: integers drawn uniformly from the inclusive range
  ``[lo, hi]``;
* lengths ``lognormal``: ``clip(rint(exp(N(ln median, sigma^2))), lo, hi)``
  with ``sigma = 0.5``.  Log-normal lengths stand in for the number of
  expressed genes per cell, which varies from hundreds to thousands
  (Sigmoid Attention for single-cell Foundation Models, section 1);
* padded length ``L``: the batch maximum, or a fixed value;
* packed documents: document lengths uniform in ``[64, 1024]`` laid end to
  end from position 0 until the sequence length is reached, the last one
  truncated; the element mask is causal within one document and zero across
  documents and on padding (the packed fine-tuning masks of Binary Block
  Masking, "Applications");
* tensors: ``standard_normal`` float32 over the full padded shape
  ``[B, H, L, d]``, rounded to bf16 with round-to-nearest-even.  Tensors are
  returned as ``uint16`` arrays holding bf16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

SIGMOID, SOFTMAX, SOFTMAX1 = 0, 1, 2
BIAS_NONE, BIAS_LOG_SEQLEN, BIAS_LOG_PADLEN = 0, 1, 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def lengths_uniform(rng: np.random.Generator, B: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def lengths_lognormal(rng: np.random.Generator, B: int, median: float, sigma: float,
                      lo: int, hi: int) -> np.ndarray:
    raw = np.exp(rng.normal(np.log(median), sigma, size=B))
    return np.clip(np.rint(raw), lo, hi).astype(np.int32)


def packed_documents(rng: np.random.Generator, n: int, lo: int = 64, hi: int = 1024) -> list:
    """Document lengths laid from position 0 until ``n``; the last one is cut."""
    docs, pos = [], 0
    while pos < n:
        length = int(rng.integers(lo, hi + 1))
        length = min(length, n - pos)
        docs.append(length)
        pos += length
    return docs


def packed_causal_mask(seq_lens: np.ndarray, docs: list, L: int) -> np.ndarray:
    """uint8 [B, L, L]: 1 where key c may be seen by query r.

    Causal (c <= r) within one document, 0 across documents and on padding.
    """
    B = len(seq_lens)
    mask = np.zeros((B, L, L), dtype=np.uint8)
    idx = np.arange(L)
    for b in range(B):
        doc_id = np.full(L, -1, dtype=np.int64)
        pos = 0
        for i, length in enumerate(docs[b]):
            doc_id[pos:pos + length] = i
            pos += length
        same = (doc_id[:, None] == doc_id[None, :]) & (doc_id[:, None] >= 0)
        causal = idx[None, :] <= idx[:, None]
        mask[b] = (same & causal).astype(np.uint8)
    return mask


def packed_causal_ranges(seq_lens: np.ndarray, docs: list, L: int) -> np.ndarray:
    """int32 [B, L, 2]: the key range [start of r's document, r] of each query
    row r < n, and the empty range (0, -1) for padded rows.  The same pattern
    as packed_causal_mask, one interval per row."""
    B = len(seq_lens)
    kr = np.zeros((B, L, 2), dtype=np.int32)
    kr[:, :, 1] = -1
    for b in range(B):
        pos = 0
        for length in docs[b]:
            rows = np.arange(pos, pos + length)
            kr[b, rows, 0] = pos
            kr[b, rows, 1] = rows
            pos += length
    return kr


def random_tensor(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


@dataclass
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    seq_lens: np.ndarray
    block_q: int
    block_k: int
    variant: int = SIGMOID
    bias: int = BIAS_LOG_SEQLEN
    mask: Optional[np.ndarray] = None
    key_range: Optional[np.ndarray] = None
    docs: Optional[list] = None
    q: Optional[np.ndarray] = None
    k: Optional[np.ndarray] = None
    v: Optional[np.ndarray] = None
    do: Optional[np.ndarray] = None
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def valid_pairs(self) -> int:
        """Number of (query, key) pairs that are attended, summed over the batch."""
        if self.mask is None:
            n = np.clip(self.seq_lens.astype(np.int64), 0, self.L)
            return int((n * n).sum())
        total = 0
        for b in range(self.B):
            n = int(np.clip(self.seq_lens[b], 0, self.L))
            total += int(self.mask[b, :n, :n].astype(np.int64).sum())
        return total


def _tensors(rng, w: Workload, names) -> None:
    shape = (w.B, w.H, w.L, w.d)
    for name in names:
        setattr(w, name, random_tensor(rng, shape))


def make_workload(name: str, *, seed: int = 0, B: int, H: int, d: int,
                  lengths: str, lo: int, hi: int, median: float = 800.0, sigma: float = 0.5,
                  L: Optional[int] = None, block_q: int = 128, block_k: int = 128,
                  variant: int = SIGMOID, bias: int = BIAS_LOG_SEQLEN,
                  docs: bool = False, tensors=("q", "k", "v"),
                  seq_lens: Optional[np.ndarray] = None) -> Workload:
    """Draw one workload.  ``L=None`` pads to the batch maximum."""
    rng = np.random.default_rng(seed)
    if seq_lens is not None:
        n = np.asarray(seq_lens, dtype=np.int32)
    elif lengths == "uniform":
        n = lengths_uniform(rng, B, lo, hi)
    elif lengths == "lognormal":
        n = lengths_lognormal(rng, B, median, sigma, lo, hi)
    else:
        raise ValueError(lengths)
    padded = int(n.max()) if L is None else int(L)
    padded = max(padded, 1)
    w = Workload(name=name, B=B, H=H, L=padded, d=d, seq_lens=n, block_q=block_q,
                 block_k=block_k, variant=variant, bias=bias, seed=seed)
    if docs:
        w.docs = [packed_documents(rng, int(min(max(x, 0), padded))) for x in n]
        w.mask = packed_causal_mask(n, w.docs, padded)
        w.key_range = packed_causal_ranges(n, w.docs, padded)
    _tensors(rng, w, tensors)
    return w


# The five benchmark workloads.  Sizes and distributions follow the text that
# describes them; sigma = 0.5 for log-normal lengths is this module's choice.
def tiny_sigmoid(seed: int = 0, tensors=("q", "k", "v")) -> Workload:
    """B4 H1 d64, lengths uniform in [16, 128] padded to 128, block 32."""
    return make_workload("tiny_sigmoid_b4h1d64_l128", seed=seed, B=4, H=1, d=64,
                         lengths="uniform", lo=16, hi=128, L=128, block_q=32, block_k=32,
                         tensors=tensors)


def single_cell(seed: int = 0, tensors=("q", "k", "v"), hi: int = 2048,
                sigma: float = 0.5) -> Workload:
    """B32 H8 d64, log-normal lengths (median 800) clipped to [200, hi]."""
    return make_workload(f"single_cell_b32h8d64_lognormal800_clip{hi}", seed=seed, B=32, H=8,
                         d=64, lengths="lognormal", lo=200, hi=hi, median=800.0, sigma=sigma,
                         block_q=128, block_k=128, tensors=tensors)


def tiny_variants(seed: int = 0, variant: int = SOFTMAX) -> Workload:
    """Tiny shapes run with the softmax, softmax_1 or sigmoid variant."""
    w = tiny_sigmoid(seed)
    w.variant = variant
    w.bias = BIAS_LOG_SEQLEN if variant == SIGMOID else BIAS_NONE
    w.name = f"tiny_variant{variant}_b4h1d64_l128"
    return w


def long_packed_docs(seed: int = 0, tensors=("q", "k", "v")) -> Workload:
    """B8 H16 d128, lengths uniform in [1024, 8192], causal packed-document mask."""
    return make_workload("long_docs_b8h16d128_causal_packed", seed=seed, B=8, H=16, d=128,
                         lengths="uniform", lo=1024, hi=8192, block_q=128, block_k=128,
                         docs=True, tensors=tensors)


def single_cell_backward(seed: int = 0) -> Workload:
    """The single-cell shapes with lengths clipped to [200, 4096], plus dO."""
    w = single_cell(seed, tensors=("q", "k", "v", "do"), hi=4096)
    w.name = "single_cell_bwd_b32h8d64_lognormal800_clip4096"
    return w
