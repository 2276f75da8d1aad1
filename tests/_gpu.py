"""Helpers for the GPU parity tests: move bf16 bit arrays to the GPU, and
compare GPU results with the oracle to the stated bounds (max abs error
<= 1e-2 and relative L2 error <= 5e-3 on valid rows; padded rows exactly 0).

The max-abs bound is stated for unit-scale outputs.  It is applied per output
row r: |got[r, i] - want[r, i]| <= 1e-2 * max(1, max_j |want[r, j]|).  Every
element of a row is a sum over the same weights, and rounding those weights
to bf16 (2^-9 relative each) moves all of them by an amount that grows with
the row's scale: sigmoid without the -ln n bias sums tens of weights near
1/2, rows reach |x| ~ 10, and a CPU model of the kernel's roundings alone
(bf16 weights, bf16 output) gives 3e-2 on an element of size 0.3 in such a
row.  A row whose values stay within 1 gets exactly the absolute bound,
whatever the other rows hold; for every benchmark workload |O| < 1."""
import sys

import numpy as np
import torch

MAX_ABS = 1e-2
REL_L2 = 5e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_gpu(x: np.ndarray, dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def gpu_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def row_valid(seq_lens, B, L):
    idx = np.arange(L)
    n = np.clip(np.asarray(seq_lens, dtype=np.int64), 0, L)
    return idx[None, :] < n[:, None]  # [B, L]


def scaled_max_abs(got: np.ndarray, want: np.ndarray) -> float:
    """max |got - want| / max(1, row scale): the row scale is max_j |want[r, j]|
    over the row's elements (the last axis of a 2-D array of rows), or |want_i|
    itself for a 1-D array.  At most MAX_ABS when every element meets its
    bound."""
    if got.size == 0:
        return 0.0
    mag = np.abs(want)
    if want.ndim >= 2:
        mag = mag.max(axis=-1, keepdims=True)
    return float((np.abs(got - want) / np.maximum(1.0, mag)).max())


def rel_l2(got: np.ndarray, want: np.ndarray) -> float:
    denom = float(np.linalg.norm(want))
    return float(np.linalg.norm(got - want) / denom) if denom > 0 else float(np.linalg.norm(got))


def assert_close(got: np.ndarray, want: np.ndarray, what: str):
    """got/want: arrays of valid rows ([rows, d]); checks both error bounds
    and returns (row-scaled max-abs figure, relative L2)."""
    if got.size == 0:
        return 0.0, 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    max_abs, rel = scaled_max_abs(got, want), rel_l2(got, want)
    assert max_abs <= MAX_ABS, f"{what}: max abs error (row-scaled) {max_abs:.3e} > {MAX_ABS}"
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    return max_abs, rel


def assert_rows(got_full: np.ndarray, want_full: np.ndarray, seq_lens, what: str):
    """[B, H, L, d] arrays: valid rows within bounds, padded rows exactly zero."""
    B, H, L, _ = got_full.shape
    valid = row_valid(seq_lens, B, L)
    vmask = np.broadcast_to(valid[:, None, :], (B, H, L))
    res = assert_close(got_full[vmask], want_full[vmask], what)
    pad = got_full[~vmask]
    assert np.all(pad == 0), f"{what}: padded rows are not exactly zero"
    return res


def decode_schedule(buf: np.ndarray, B: int, H: int, L: int, block_q: int, block_k: int) -> dict:
    """The schedule buffer blockmask_build writes, in oracle.schedule's form.
    Layout (include/sigattn.h): items1 then items2, 16 bytes per slot
    {b, h, tile | kind << 30, n} (tile -1 past the last item), then per batch
    entry and 128-row group the query lists (count, then e | kept << 24 |
    full << 28 per entry; 1 + Tk words each) and the key lists (1 + Tq)."""
    G = -(-L // 128)
    Tq, Tk = -(-L // block_q), -(-L // block_k)
    slots1 = 8 * (-(-(B * H) // 8)) * G
    words = np.frombuffer(np.ascontiguousarray(buf).tobytes(), dtype=np.int32)
    out = {}
    pos = 0
    for name, nslots in (("items1", slots1), ("items2", 2 * slots1)):
        it = words[pos:pos + 4 * nslots].reshape(nslots, 4)
        out[name] = [None if z < 0 else (int(b), int(h), int(z) >> 30, int(z) & 0x3fffffff, int(n))
                     for b, h, z, n in it]
        pos += 4 * nslots
    for name, stride in (("qlists", 1 + Tk), ("klists", 1 + Tq)):
        lists = words[pos:pos + B * G * stride].reshape(B, G, stride).view(np.uint32)
        out[name] = [[[(int(w & 0xffffff), int((w >> 24) & 15), int(w >> 28))
                       for w in lists[b, g, 1:1 + lists[b, g, 0]]] for g in range(G)]
                     for b in range(B)]
        pos += B * G * stride
    assert 4 * pos <= buf.size
    return out
