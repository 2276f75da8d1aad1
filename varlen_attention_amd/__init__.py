"""varlen_attention_amd: fused, tiled attention over padded variable-length
batches on AMD MI355X (gfx950).

Thin Python binding of ``libsigattn.so`` (C ABI in ``include/sigattn.h``).
Every function here only marshals arguments: it takes torch tensors that
already live on the GPU, checks their dtypes, devices and layouts, and calls
the C entry point of the same name on torch's current stream.  All
computation happens in the HIP kernels; there is no CPU or PyTorch fallback,
and the import fails loudly if the library has not been built
(``python -m varlen_attention_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

SIGMOID, SOFTMAX, SOFTMAX1 = 0, 1, 2
BIAS_NONE, BIAS_LOG_SEQLEN, BIAS_LOG_PADLEN = 0, 1, 2
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_LAUNCH = 0, -1, -2, -3, -4
# Longest padded length accepted together with an element mask (SIGATTN_MAX_MASKED_L).
MAX_MASKED_L = 46080

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsigattn.so")
EXPORTS = ("blockmask_build", "sigattn_schedule_bytes", "sigattn_fwd", "sigattn_fwd_noalloc",
           "sigattn_bwd", "sigattn_bwd_dkdv", "sigattn_bwd_dq", "sigattn_diff_fwd",
           "sigattn_diff_bwd", "sigattn_last_error")
# Bytes of the library's own schedule memory for sigattn_fwd_noalloc
# (SIGATTN_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024


class SigattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
        ("stride_l", ctypes.c_int64),
        ("o_stride_b", ctypes.c_int64), ("o_stride_h", ctypes.c_int64),
        ("o_stride_l", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsigattn.so and declare its signatures (no GPU needed)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m varlen_attention_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int32
    S = ctypes.POINTER(Shape)
    I64 = ctypes.c_int64
    lib.sigattn_schedule_bytes.argtypes = [I, I, I, I, I, I]
    lib.sigattn_schedule_bytes.restype = I64
    lib.blockmask_build.argtypes = [P, P, P, I, I, I, I, I, P, P, I64, P]
    lib.blockmask_build.restype = ctypes.c_int
    lib.sigattn_fwd.argtypes = [S, P, P, P, P, P, P, P, P, I, I, P, P, P]
    lib.sigattn_fwd.restype = ctypes.c_int
    lib.sigattn_fwd_noalloc.argtypes = [S, P, P, P, P, P, P, P, I, I, P, P, P]
    lib.sigattn_fwd_noalloc.restype = ctypes.c_int
    lib.sigattn_bwd.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, I, I, P, P, P, P]
    lib.sigattn_bwd.restype = ctypes.c_int
    lib.sigattn_bwd_dkdv.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, I, I, P, P, P]
    lib.sigattn_bwd_dkdv.restype = ctypes.c_int
    lib.sigattn_bwd_dq.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, I, I, P, P]
    F = ctypes.c_float
    lib.sigattn_diff_fwd.argtypes = [S, P, P, P, P, P, P, P, P, P, P, I, F, P, P, P, P, P, P]
    lib.sigattn_diff_fwd.restype = ctypes.c_int
    lib.sigattn_diff_bwd.argtypes = [S] + [P] * 15 + [I, F] + [P] * 6
    lib.sigattn_diff_bwd.restype = ctypes.c_int
    lib.sigattn_bwd_dq.restype = ctypes.c_int
    lib.sigattn_last_error.argtypes = []
    lib.sigattn_last_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != OK:
        msg = load_library().sigattn_last_error().decode()
        raise SigattnError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")


def _lens(seq_lens: torch.Tensor, B: int, device) -> None:
    """seq_lens: int32 [B] on the same GPU as the tensors it describes (the
    kernels read seq_lens[0 .. B-1], so a shorter tensor would be read past
    its end)."""
    _need(seq_lens, "seq_lens", torch.int32)
    if seq_lens.dim() != 1 or seq_lens.shape[0] != B:
        raise ValueError(f"seq_lens must be a 1-D tensor of B = {B} lengths "
                         f"(got shape {tuple(seq_lens.shape)})")
    if device is not None and seq_lens.device != device:
        raise ValueError(f"seq_lens is on {seq_lens.device}, the tensors on {device}")


def _layout(ts, names):
    """All tensors [B, H, L, d] with equal strides and unit stride in d."""
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError(f"{names[0]} must be [B, H, L, d]")
    for t, nm in zip(ts, names):
        if t.shape != ref.shape:
            raise ValueError(f"{nm} has shape {tuple(t.shape)}, expected {tuple(ref.shape)}")
        if t.stride() != ref.stride():
            raise ValueError(f"{nm} strides {t.stride()} differ from {names[0]} {ref.stride()}")
        if t.stride(3) != 1:
            raise ValueError(f"{nm} must be contiguous along the head dimension")
    return ref.stride()


def _shape(q: torch.Tensor, out_strides, scale, block_q, block_k) -> Shape:
    B, H, L, d = q.shape
    s = q.stride()
    return Shape(B, H, L, d, s[0], s[1], s[2], out_strides[0], out_strides[1], out_strides[2],
                 float(scale) if scale is not None else 0.0, block_q, block_k)


def num_tiles(L: int, block: int) -> int:
    return -(-L // block)


def _key_range(key_range, B, L):
    if key_range is not None:
        _need(key_range, "key_range", torch.int32)
        if tuple(key_range.shape) != (B, L, 2) or not key_range.is_contiguous():
            raise ValueError("key_range must be a contiguous int32 [B, L, 2] tensor")


def schedule_bytes(B: int, H: int, L: int, block_q: int = 128, block_k: int = 128,
                   dense_mask: bool = False) -> int:
    """Bytes of the schedule buffer blockmask_build fills (sigattn_schedule_bytes);
    ``dense_mask``: for a batch with an element mask (the schedule then also
    holds the mask packed to bits)."""
    nbytes = load_library().sigattn_schedule_bytes(B, H, L, block_q, block_k, int(dense_mask))
    _check(int(nbytes) if nbytes < 0 else OK)
    return int(nbytes)


def _schedule(schedule, block_mask, mask=None, dims=None):
    """Checks a schedule argument; with a mask (dims = B, H, L, block_q,
    block_k) the schedule must hold the packed mask, which only a schedule
    built with that mask does."""
    if schedule is not None:
        _need(schedule, "schedule", torch.uint8)
        if schedule.dim() != 1 or not schedule.is_contiguous():
            raise ValueError("schedule must be a contiguous 1-D uint8 tensor")
        if block_mask is None:
            raise ValueError("a schedule needs the block mask it was built with")
        if mask is not None and dims is not None:
            need = schedule_bytes(*dims, dense_mask=True)
            if schedule.numel() < need:
                raise ValueError(f"with a mask the schedule must be one built with it "
                                 f"({need} bytes, got {schedule.numel()})")


def blockmask_build(seq_lens: torch.Tensor, L: int, block_q: int = 128, block_k: int = 128,
                    mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    stream=None, key_range: Optional[torch.Tensor] = None,
                    heads: Optional[int] = None, schedule: Optional[torch.Tensor] = None):
    """Block matrix uint8 [B, ceil(L/block_q), ceil(L/block_k)] on the GPU: bit 0
    the binary block mask, bit 1 full tiles.  The element mask is ``mask``
    (uint8 [B, L, L]) or ``key_range`` (int32 [B, L, 2]: row r keeps keys
    lo..hi), not both.

    With ``heads`` (the H of the attention calls) it also builds the work
    schedule (into ``schedule``, a uint8 tensor of ``schedule_bytes(...)``
    bytes, allocated when not given) and returns ``(block_mask, schedule)``;
    pass both to the attention calls of this batch."""
    _need(seq_lens, "seq_lens", torch.int32)
    if seq_lens.dim() != 1:
        raise ValueError(f"seq_lens must be a 1-D tensor (got shape {tuple(seq_lens.shape)})")
    B = seq_lens.shape[0]
    if mask is not None:
        _need(mask, "mask", torch.uint8)
        if tuple(mask.shape) != (B, L, L) or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8 [B, L, L] tensor")
    _key_range(key_range, B, L)
    shape = (B, num_tiles(L, block_q), num_tiles(L, block_k))
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=seq_lens.device)
    elif tuple(out.shape) != shape or out.dtype != torch.uint8 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous uint8 tensor of shape {shape}")
    if schedule is not None and heads is None:
        raise ValueError("building a schedule needs the number of heads")
    nbytes = 0
    if heads is not None:
        nbytes = schedule_bytes(B, heads, L, block_q, block_k, dense_mask=mask is not None)
        if schedule is None:
            schedule = torch.empty(nbytes, dtype=torch.uint8, device=seq_lens.device)
        _schedule(schedule, out)
        if schedule.numel() < nbytes:
            raise ValueError(f"schedule holds {schedule.numel()} bytes, {nbytes} needed")
    lib = load_library()
    _check(lib.blockmask_build(_ptr(seq_lens.contiguous()), _ptr(mask), _ptr(key_range), B,
                               heads or 0, L, block_q, block_k, _ptr(out), _ptr(schedule),
                               nbytes if schedule is not None else 0, _stream(stream)))
    return out if heads is None else (out, schedule)


def sigattn_fwd(q, k, v, seq_lens, block_mask=None, mask=None, bias=BIAS_LOG_SEQLEN,
                variant=SIGMOID, scale=None, block_q=128, block_k=128, out=None, lse=None,
                return_lse=False, stream=None, key_range=None, schedule=None):
    """Forward pass.  q, k, v: bf16 [B, H, L, d] on the GPU (equal strides).

    Returns o (bf16, same shape) or (o, lse) with ``return_lse=True``.
    """
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16)
    _layout([q, k, v], ["q", "k", "v"])
    _lens(seq_lens, q.shape[0], q.device)
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _need(out, "out", torch.bfloat16)
    if tuple(out.shape) != tuple(q.shape) or out.stride(3) != 1:
        raise ValueError("out must match q's shape with unit stride in d")
    B, H, L, d = q.shape
    if (return_lse or lse is not None) and lse is None:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, H, L] tensor")
    if mask is not None:
        _need(mask, "mask", torch.uint8)
        if tuple(mask.shape) != (B, L, L) or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8 [B, L, L] tensor")
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8)
        want = (B, num_tiles(L, block_q), num_tiles(L, block_k))
        if tuple(block_mask.shape) != want or not block_mask.is_contiguous():
            raise ValueError(f"block_mask must be a contiguous uint8 tensor of shape {want}")
    _key_range(key_range, B, L)
    _schedule(schedule, block_mask, mask, (B, H, L, block_q, block_k))
    shape = _shape(q, out.stride(), scale, block_q, block_k)
    lib = load_library()
    _check(lib.sigattn_fwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v),
                           _ptr(seq_lens.contiguous()), _ptr(block_mask), _ptr(schedule),
                           _ptr(mask), _ptr(key_range), bias, variant, _ptr(out), _ptr(lse),
                           _stream(stream)))
    return (out, lse) if return_lse else out


def sigattn_fwd_noalloc(q, k, v, seq_lens, block_mask, out, lse=None, mask=None,
                        bias=BIAS_LOG_SEQLEN, variant=SIGMOID, scale=None, block_q=128,
                        block_k=128, stream=None, key_range=None):
    """sigattn_fwd with the work schedule kept in the library's own device
    memory (sigattn_fwd_noalloc): allocates nothing, so the output ``out`` (and
    ``lse``, when wanted) must be given.  block_mask is required."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, nm, torch.bfloat16)
    _layout([q, k, v], ["q", "k", "v"])
    _lens(seq_lens, q.shape[0], q.device)
    if not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous")
    if tuple(out.shape) != tuple(q.shape) or out.stride(3) != 1:
        raise ValueError("out must match q's shape with unit stride in d")
    B, H, L, d = q.shape
    if lse is not None:
        _need(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, H, L] tensor")
    if block_mask is None:
        raise ValueError("sigattn_fwd_noalloc needs the block mask")
    _need(block_mask, "block_mask", torch.uint8)
    want = (B, num_tiles(L, block_q), num_tiles(L, block_k))
    if tuple(block_mask.shape) != want or not block_mask.is_contiguous():
        raise ValueError(f"block_mask must be a contiguous uint8 tensor of shape {want}")
    if mask is not None:
        _need(mask, "mask", torch.uint8)
        if tuple(mask.shape) != (B, L, L) or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8 [B, L, L] tensor")
    _key_range(key_range, B, L)
    shape = _shape(q, out.stride(), scale, block_q, block_k)
    _check(load_library().sigattn_fwd_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens), _ptr(block_mask),
        _ptr(mask), _ptr(key_range), bias, variant, _ptr(out), _ptr(lse), _stream(stream)))
    return out


def _bwd_args(q, k, v, dout, seq_lens, block_mask, mask, grads, block_q, block_k, variant, o,
              lse, key_range, schedule=None):
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _need(t, nm, torch.bfloat16)
    _layout([q, k, v, dout], ["q", "k", "v", "dout"])
    _lens(seq_lens, q.shape[0], q.device)
    outs = [torch.empty_like(q, memory_format=torch.contiguous_format) if g is None else g
            for g in grads]
    for g in outs:
        _need(g, "gradient output", torch.bfloat16)
    _layout(outs, ["gradient output"] * len(outs))
    B, H, L, d = q.shape
    if variant != SIGMOID:
        if o is None or lse is None:
            raise ValueError("the softmax-variant backward needs the forward's o and lse")
    if o is not None:
        _need(o, "o", torch.bfloat16)
        if tuple(o.shape) != tuple(q.shape) or o.stride() != outs[0].stride():
            raise ValueError("o must have q's shape and the gradient outputs' strides")
    if lse is not None:
        _need(lse, "lse", torch.float32)
        if tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous fp32 [B, H, L] tensor")
    if mask is not None:
        _need(mask, "mask", torch.uint8)
        if tuple(mask.shape) != (B, L, L) or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8 [B, L, L] tensor")
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8)
        want = (B, num_tiles(L, block_q), num_tiles(L, block_k))
        if tuple(block_mask.shape) != want or not block_mask.is_contiguous():
            raise ValueError(f"block_mask must be a contiguous uint8 tensor of shape {want}")
    _key_range(key_range, B, L)
    _schedule(schedule, block_mask, mask, (B, H, L, block_q, block_k))
    return outs


def sigattn_bwd(q, k, v, dout, seq_lens, block_mask=None, mask=None, bias=BIAS_LOG_SEQLEN,
                variant=SIGMOID, scale=None, block_q=128, block_k=128, dq=None, dk=None,
                dv=None, o=None, lse=None, stream=None, key_range=None, schedule=None):
    """Gradients (dq, dk, dv) of sum(dout * o); bf16 [B, H, L, d] on the GPU.

    The softmax variants need the forward's output ``o`` and ``lse`` (from
    ``sigattn_fwd(..., return_lse=True)`` with the same variant and bias).
    One launch for the dK/dV and dQ work when their tile heights agree (see
    include/sigattn.h); results equal sigattn_bwd_dkdv + sigattn_bwd_dq."""
    dq, dk, dv = _bwd_args(q, k, v, dout, seq_lens, block_mask, mask, (dq, dk, dv), block_q,
                           block_k, variant, o, lse, key_range, schedule)
    shape = _shape(q, dq.stride(), scale, block_q, block_k)
    _check(load_library().sigattn_bwd(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(o), _ptr(lse),
        _ptr(seq_lens.contiguous()), _ptr(block_mask), _ptr(schedule), _ptr(mask),
        _ptr(key_range), bias, variant, _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)))
    return dq, dk, dv


def sigattn_bwd_dkdv(q, k, v, dout, seq_lens, block_mask=None, mask=None, bias=BIAS_LOG_SEQLEN,
                     variant=SIGMOID, scale=None, block_q=128, block_k=128, dk=None, dv=None,
                     o=None, lse=None, stream=None, key_range=None, schedule=None):
    """The dK/dV half of the backward pass (one kernel): returns (dk, dv)."""
    dk, dv = _bwd_args(q, k, v, dout, seq_lens, block_mask, mask, (dk, dv), block_q, block_k,
                       variant, o, lse, key_range, schedule)
    shape = _shape(q, dk.stride(), scale, block_q, block_k)
    _check(load_library().sigattn_bwd_dkdv(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(o), _ptr(lse),
        _ptr(seq_lens.contiguous()), _ptr(block_mask), _ptr(schedule), _ptr(mask),
        _ptr(key_range), bias, variant, _ptr(dk), _ptr(dv), _stream(stream)))
    return dk, dv


def sigattn_bwd_dq(q, k, v, dout, seq_lens, block_mask=None, mask=None, bias=BIAS_LOG_SEQLEN,
                   variant=SIGMOID, scale=None, block_q=128, block_k=128, dq=None, o=None,
                   lse=None, stream=None, key_range=None, schedule=None):
    """The dQ half of the backward pass (one kernel): returns dq."""
    (dq,) = _bwd_args(q, k, v, dout, seq_lens, block_mask, mask, (dq,), block_q, block_k,
                      variant, o, lse, key_range, schedule)
    shape = _shape(q, dq.stride(), scale, block_q, block_k)
    _check(load_library().sigattn_bwd_dq(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(o), _ptr(lse),
        _ptr(seq_lens.contiguous()), _ptr(block_mask), _ptr(schedule), _ptr(mask),
        _ptr(key_range), bias, variant, _ptr(dq), _stream(stream)))
    return dq

def sigattn_diff_fwd(q1, k1, q2, k2, v, seq_lens, lam: float, block_mask=None, mask=None,
                     key_range=None, bias=BIAS_NONE, scale=None, block_q=128, block_k=128,
                     out=None, lse1=None, lse2=None, return_lse=False, stream=None,
                     o1=None, o2=None, return_maps=False, schedule=None):
    """Differential attention forward: (softmax(S1) - lam softmax(S2)) V, both
    maps in one tile loop.  q1, k1, q2, k2, v: bf16 [B, H, L, d] on the GPU
    with equal strides.  Returns o, or (o, lse1, lse2) with return_lse=True;
    with return_maps=True also each map's own output: (o, lse1, lse2, o1, o2)
    (what sigattn_diff_bwd needs)."""
    for t, nm in ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v")):
        _need(t, nm, torch.bfloat16)
    _layout([q1, k1, q2, k2, v], ["q1", "k1", "q2", "k2", "v"])
    _lens(seq_lens, q1.shape[0], q1.device)
    if out is None:
        out = torch.empty_like(q1, memory_format=torch.contiguous_format)
    _need(out, "out", torch.bfloat16)
    if tuple(out.shape) != tuple(q1.shape) or out.stride(3) != 1:
        raise ValueError("out must match q1's shape with unit stride in d")
    B, H, L, d = q1.shape
    lses = []
    for l_ in (lse1, lse2):
        if return_lse and l_ is None:
            l_ = torch.empty((B, H, L), dtype=torch.float32, device=q1.device)
        if l_ is not None:
            _need(l_, "lse", torch.float32)
            if tuple(l_.shape) != (B, H, L) or not l_.is_contiguous():
                raise ValueError("lse1/lse2 must be contiguous float32 [B, H, L] tensors")
        lses.append(l_)
    if mask is not None:
        _need(mask, "mask", torch.uint8)
        if tuple(mask.shape) != (B, L, L) or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8 [B, L, L] tensor")
    _key_range(key_range, B, L)
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8)
        want = (B, num_tiles(L, block_q), num_tiles(L, block_k))
        if tuple(block_mask.shape) != want or not block_mask.is_contiguous():
            raise ValueError(f"block_mask must be a contiguous uint8 tensor of shape {want}")
    if return_maps:
        return_lse = True
        lses = [torch.empty((B, H, L), dtype=torch.float32, device=q1.device) if l_ is None
                else l_ for l_ in lses]
        o1 = torch.empty_like(out) if o1 is None else o1
        o2 = torch.empty_like(out) if o2 is None else o2
    for om in (o1, o2):
        if om is not None:
            _need(om, "o1/o2", torch.bfloat16)
            if tuple(om.shape) != tuple(out.shape) or om.stride() != out.stride():
                raise ValueError("o1 and o2 must have out's shape and strides")
    _schedule(schedule, block_mask, mask, (B, H, L, block_q, block_k))
    shape = _shape(q1, out.stride(), scale, block_q, block_k)
    _check(load_library().sigattn_diff_fwd(
        ctypes.byref(shape), _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v),
        _ptr(seq_lens.contiguous()), _ptr(block_mask), _ptr(schedule), _ptr(mask),
        _ptr(key_range), bias, float(lam), _ptr(out), _ptr(o1), _ptr(o2), _ptr(lses[0]),
        _ptr(lses[1]), _stream(stream)))
    if return_maps:
        return out, lses[0], lses[1], o1, o2
    return (out, lses[0], lses[1]) if return_lse else out


def sigattn_diff_bwd(q1, k1, q2, k2, v, dout, o1, o2, lse1, lse2, seq_lens, lam: float,
                     block_mask=None, mask=None, key_range=None, bias=BIAS_NONE, scale=None,
                     block_q=128, block_k=128, grads=None, stream=None, schedule=None):
    """Gradients (dq1, dk1, dq2, dk2, dv) of sum(dout * o) for the differential
    forward; o1, o2, lse1, lse2 from sigattn_diff_fwd(..., return_maps=True)."""
    for t, nm in ((q1, "q1"), (k1, "k1"), (q2, "q2"), (k2, "k2"), (v, "v"), (dout, "dout")):
        _need(t, nm, torch.bfloat16)
    _layout([q1, k1, q2, k2, v, dout], ["q1", "k1", "q2", "k2", "v", "dout"])
    _lens(seq_lens, q1.shape[0], q1.device)
    outs = [torch.empty_like(q1, memory_format=torch.contiguous_format) for _ in range(5)] \
        if grads is None else list(grads)
    for g_ in outs:
        _need(g_, "gradient output", torch.bfloat16)
    _layout(outs, ["gradient output"] * 5)
    B, H, L, d = q1.shape
    for om in (o1, o2):
        _need(om, "o1/o2", torch.bfloat16)
        if tuple(om.shape) != tuple(q1.shape) or om.stride() != outs[0].stride():
            raise ValueError("o1 and o2 must have q1's shape and the gradient outputs' strides")
    for l_ in (lse1, lse2):
        _need(l_, "lse", torch.float32)
        if tuple(l_.shape) != (B, H, L) or not l_.is_contiguous():
            raise ValueError("lse1/lse2 must be contiguous float32 [B, H, L] tensors")
    if mask is not None:
        _need(mask, "mask", torch.uint8)
        if tuple(mask.shape) != (B, L, L) or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous uint8 [B, L, L] tensor")
    _key_range(key_range, B, L)
    if block_mask is not None:
        _need(block_mask, "block_mask", torch.uint8)
        want = (B, num_tiles(L, block_q), num_tiles(L, block_k))
        if tuple(block_mask.shape) != want or not block_mask.is_contiguous():
            raise ValueError(f"block_mask must be a contiguous uint8 tensor of shape {want}")
    _schedule(schedule, block_mask, mask, (B, H, L, block_q, block_k))
    shape = _shape(q1, outs[0].stride(), scale, block_q, block_k)
    _check(load_library().sigattn_diff_bwd(
        ctypes.byref(shape), _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), _ptr(v), _ptr(dout),
        _ptr(o1), _ptr(o2), _ptr(lse1), _ptr(lse2), _ptr(seq_lens.contiguous()),
        _ptr(block_mask), _ptr(schedule), _ptr(mask), _ptr(key_range), bias, float(lam),
        *(_ptr(g_) for g_ in outs), _stream(stream)))
    return tuple(outs)
