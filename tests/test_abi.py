"""The C-ABI library loads on the CPU, exports every function that
include/sigattn.h declares, and rejects bad arguments on the host before
anything reaches the GPU (none of these calls launches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sigattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def lib():
    import varlen_attention_amd as va
    if not os.path.exists(va.LIB_PATH):
        pytest.fail("libsigattn.so is not built (python -m varlen_attention_amd.build)")
    return va.load_library()


def test_header_declares_the_boundary():
    import varlen_attention_amd as va
    assert declared_functions() == sorted(
        ["blockmask_build", "sigattn_schedule_bytes", "sigattn_fwd", "sigattn_fwd_noalloc",
         "sigattn_bwd", "sigattn_bwd_dkdv", "sigattn_bwd_dq", "sigattn_diff_bwd",
         "sigattn_diff_fwd", "sigattn_last_error"])
    assert sorted(va.EXPORTS) == declared_functions()


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def _shape(va, **kw):
    base = dict(B=2, H=2, L=100, d=64, stride_b=2 * 100 * 64, stride_h=100 * 64, stride_l=64,
                o_stride_b=0, o_stride_h=0, o_stride_l=0, scale=0.0, block_q=128, block_k=128)
    base.update(kw)
    return va.Shape(**base)


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails first


def _fwd(lib, va, shape, q=FAKE, k=FAKE, v=FAKE, seq=FAKE, bm=None, mask=None, bias=1, var=0,
         o=FAKE, lse=None, kr=None, sched=None):
    return lib.sigattn_fwd(ctypes.byref(shape) if shape is not None else None, q, k, v, seq, bm,
                           sched, mask, kr, bias, var, o, lse, None)


def test_forward_argument_errors(lib):
    import varlen_attention_amd as va
    assert _fwd(lib, va, None) == va.ERR_INVALID_ARG
    assert b"shape" in lib.sigattn_last_error()
    assert _fwd(lib, va, _shape(va, d=96)) == va.ERR_UNSUPPORTED
    assert _fwd(lib, va, _shape(va, B=0)) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va, block_q=48)) == va.ERR_UNSUPPORTED
    # Too many workgroups for one launch: 16 * ceil(B * H / 8) * ceil(L / 128)
    # must stay below 2^24 (times 256 threads, HIP's 32-bit grid).
    assert _fwd(lib, va, _shape(va, B=65535, H=1024, L=10000)) == va.ERR_UNSUPPORTED
    at_limit = 128 * (1 << 20)  # B * H = 8: 16 * 1 * 2^20 workgroups = 2^24
    assert _fwd(lib, va, _shape(va, B=8, H=1, L=at_limit)) == va.ERR_UNSUPPORTED
    # One tile less passes the size check and stops at the next one (null q).
    assert _fwd(lib, va, _shape(va, B=8, H=1, L=at_limit - 128), q=None) == va.ERR_INVALID_ARG
    # L near INT32_MAX: the tile count is computed without overflow.
    assert _fwd(lib, va, _shape(va, B=1, H=1, L=2**31 - 1)) == va.ERR_UNSUPPORTED
    assert b"too large" in lib.sigattn_last_error()
    assert _fwd(lib, va, _shape(va), q=None) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va), seq=None) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va), o=None) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va), bias=7) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va), var=5) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va), mask=FAKE) == va.ERR_INVALID_ARG  # mask needs block mask
    assert _fwd(lib, va, _shape(va), k=ctypes.c_void_p(0x10008)) == va.ERR_ALIGNMENT
    assert _fwd(lib, va, _shape(va, stride_l=68)) == va.ERR_ALIGNMENT
    assert _fwd(lib, va, _shape(va, stride_l=32)) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va), lse=ctypes.c_void_p(0x10002)) == va.ERR_ALIGNMENT
    # An element mask bounds L (32-bit offsets into each L x L mask).
    assert _fwd(lib, va, _shape(va, L=va.MAX_MASKED_L + 1), mask=FAKE, bm=FAKE) == va.ERR_UNSUPPORTED
    # Row strides above the 32-bit tile addressing limit.
    assert _fwd(lib, va, _shape(va, stride_l=4194304 + 8)) == va.ERR_UNSUPPORTED
    # Key ranges: not with a dense mask, only with a block mask, 8-byte aligned.
    assert _fwd(lib, va, _shape(va), mask=FAKE, kr=FAKE, bm=FAKE) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va), kr=FAKE) == va.ERR_INVALID_ARG
    assert _fwd(lib, va, _shape(va), kr=ctypes.c_void_p(0x10004), bm=FAKE) == va.ERR_ALIGNMENT
    # A schedule needs the block mask it was built with, and 16-byte alignment.
    assert _fwd(lib, va, _shape(va), sched=FAKE) == va.ERR_INVALID_ARG
    assert b"schedule" in lib.sigattn_last_error()
    assert _fwd(lib, va, _shape(va), sched=ctypes.c_void_p(0x10008), bm=FAKE) == va.ERR_ALIGNMENT


def test_noalloc_forward_argument_errors(lib):
    """sigattn_fwd_noalloc: as sigattn_fwd, plus a required block mask and a
    schedule no larger than the library's array; all checked before any HIP
    call (none of these reaches the GPU)."""
    import varlen_attention_amd as va

    def fwd0(shape, bm=FAKE, q=FAKE, mask=None, kr=None):
        return lib.sigattn_fwd_noalloc(ctypes.byref(shape), q, FAKE, FAKE, FAKE, bm, mask, kr, 1,
                                       0, FAKE, None, None)

    assert fwd0(_shape(va), bm=None) == va.ERR_INVALID_ARG
    assert b"block mask" in lib.sigattn_last_error()
    assert fwd0(_shape(va), q=None) == va.ERR_INVALID_ARG
    assert fwd0(_shape(va, d=96)) == va.ERR_UNSUPPORTED
    # B32 H64 L65536: a schedule of ~50 MB, beyond the 8 MiB the library holds.
    big = _shape(va, B=32, H=64, L=65536, stride_b=64 * 65536 * 64, stride_h=65536 * 64)
    assert lib.sigattn_schedule_bytes(32, 64, 65536, 128, 128, 0) > va.NOALLOC_SCRATCH_BYTES
    assert fwd0(big) == va.ERR_UNSUPPORTED
    assert b"holds" in lib.sigattn_last_error()
    hdr = open(HEADER).read()
    m = re.search(r"#define\s+SIGATTN_NOALLOC_SCRATCH_BYTES\s+\((\d+) \* 1024 \* 1024\)", hdr)
    assert m and int(m.group(1)) * 1024 * 1024 == va.NOALLOC_SCRATCH_BYTES


def test_backward_argument_errors(lib):
    import varlen_attention_amd as va
    sh = _shape(va)
    args = [FAKE] * 4  # q, k, v, dout

    def bwd(shape=sh, o=None, lse=None, var=0, dk=FAKE, bm=None, mask=None, kr=None, sched=None):
        return lib.sigattn_bwd(ctypes.byref(shape), *args, o, lse, FAKE, bm, sched, mask, kr, 1,
                               var, FAKE, dk, FAKE, None)

    # The softmax variants need the forward's o and lse; SIGMOID ignores them.
    assert bwd(var=1) == va.ERR_INVALID_ARG
    assert bwd(var=2, o=FAKE) == va.ERR_INVALID_ARG
    assert bwd(var=1, o=ctypes.c_void_p(0x10008), lse=FAKE) == va.ERR_ALIGNMENT
    assert bwd(var=2, o=FAKE, lse=ctypes.c_void_p(0x10002)) == va.ERR_ALIGNMENT
    assert bwd(dk=None) == va.ERR_INVALID_ARG
    assert bwd(mask=FAKE) == va.ERR_INVALID_ARG  # an element mask needs its block mask
    assert bwd(shape=_shape(va, L=50000), mask=FAKE, bm=FAKE) == va.ERR_UNSUPPORTED
    assert bwd(shape=_shape(va, d=128, L=0)) == va.ERR_INVALID_ARG
    assert bwd(mask=FAKE, kr=FAKE, bm=FAKE) == va.ERR_INVALID_ARG
    assert bwd(kr=FAKE) == va.ERR_INVALID_ARG
    assert bwd(kr=ctypes.c_void_p(0x10004), bm=FAKE) == va.ERR_ALIGNMENT
    assert bwd(sched=FAKE) == va.ERR_INVALID_ARG  # a schedule needs its block mask
    assert lib.sigattn_bwd_dq(ctypes.byref(sh), *args, None, None, FAKE, None, None, None, None,
                              1, 1, FAKE, None) == va.ERR_INVALID_ARG
    assert lib.sigattn_bwd_dkdv(ctypes.byref(sh), *args, None, None, FAKE, None, None, None, None,
                                1, 0, FAKE, None, None) == va.ERR_INVALID_ARG
    assert lib.sigattn_bwd_dkdv(ctypes.byref(sh), *args, None, None, FAKE, None, FAKE, None, None,
                                1, 0, FAKE, FAKE, None) == va.ERR_INVALID_ARG


def test_diff_forward_argument_errors(lib):
    import varlen_attention_amd as va
    sh = _shape(va)

    def diff(shape=sh, q2=FAKE, lam=0.5, lse2=None, mask=None, kr=None, bm=None, o1=None):
        return lib.sigattn_diff_fwd(ctypes.byref(shape), FAKE, FAKE, q2, FAKE, FAKE, FAKE, bm,
                                    None, mask, kr, 0, lam, FAKE, o1, None, None, lse2, None)

    assert diff(q2=None) == va.ERR_INVALID_ARG
    assert diff(lam=float("nan")) == va.ERR_INVALID_ARG
    assert diff(lam=float("inf")) == va.ERR_INVALID_ARG
    assert diff(lse2=ctypes.c_void_p(0x10002)) == va.ERR_ALIGNMENT
    assert diff(q2=ctypes.c_void_p(0x10008)) == va.ERR_ALIGNMENT
    assert diff(shape=_shape(va, d=96)) == va.ERR_UNSUPPORTED
    assert diff(mask=FAKE) == va.ERR_INVALID_ARG  # mask needs its block mask
    assert diff(o1=ctypes.c_void_p(0x10008)) == va.ERR_ALIGNMENT


def test_diff_backward_argument_errors(lib):
    import varlen_attention_amd as va
    sh = _shape(va)

    def dbwd(lam=0.5, o2=FAKE, lse2=FAKE, dq2=FAKE, o1=FAKE, dv=FAKE):
        return lib.sigattn_diff_bwd(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, o1, o2,
                                    FAKE, lse2, FAKE, None, None, None, None, 0, lam, FAKE, FAKE,
                                    dq2, FAKE, dv, None)

    assert dbwd(lam=float("nan")) == va.ERR_INVALID_ARG
    assert dbwd(o2=None) == va.ERR_INVALID_ARG
    assert dbwd(dq2=None) == va.ERR_INVALID_ARG
    assert dbwd(dv=None) == va.ERR_INVALID_ARG
    assert dbwd(lse2=ctypes.c_void_p(0x10002)) == va.ERR_ALIGNMENT
    assert dbwd(o2=ctypes.c_void_p(0x10008)) == va.ERR_ALIGNMENT
    assert dbwd(o1=None) == va.ERR_INVALID_ARG  # map 1 needs its output too


def test_blockmask_argument_errors(lib):
    import varlen_attention_amd as va

    def bmb(seq=FAKE, mask=None, kr=None, B=2, H=1, L=100, bq=32, bk=32, out=FAKE, sched=None,
            nbytes=0):
        return lib.blockmask_build(seq, mask, kr, B, H, L, bq, bk, out, sched, nbytes, None)

    assert bmb(seq=None) == va.ERR_INVALID_ARG
    assert bmb(out=None) == va.ERR_INVALID_ARG
    assert bmb(B=0) == va.ERR_INVALID_ARG
    assert bmb(bq=16) == va.ERR_UNSUPPORTED
    assert bmb(mask=ctypes.c_void_p(0x10001)) == va.ERR_ALIGNMENT
    assert bmb(mask=FAKE, kr=FAKE) == va.ERR_INVALID_ARG
    assert bmb(kr=ctypes.c_void_p(0x10004)) == va.ERR_ALIGNMENT
    # With a schedule: H > 0, a 16-byte aligned buffer of at least the size.
    need = lib.sigattn_schedule_bytes(2, 3, 100, 32, 32, 0)
    assert need > 0
    assert bmb(H=0, sched=FAKE, nbytes=need) == va.ERR_INVALID_ARG
    assert bmb(H=3, sched=FAKE, nbytes=need - 1) == va.ERR_INVALID_ARG
    assert b"needed" in lib.sigattn_last_error()
    assert bmb(H=3, sched=ctypes.c_void_p(0x10008), nbytes=need) == va.ERR_ALIGNMENT
    # A batch with a mask needs the larger schedule (it carries the packed mask).
    need_m = lib.sigattn_schedule_bytes(2, 3, 100, 32, 32, 1)
    assert need_m > need
    assert bmb(mask=FAKE, H=3, sched=FAKE, nbytes=need) == va.ERR_INVALID_ARG
    assert b"needed" in lib.sigattn_last_error()
    assert bmb(B=8, H=1, L=128 << 20, sched=FAKE, nbytes=1 << 40) == va.ERR_UNSUPPORTED


def test_schedule_bytes_follow_the_layout(lib):
    """48 bytes per 128-row tile slot of the two item arrays ((batch entry,
    head) pairs rounded up to 8), plus the count and entry words of every
    query and key group; for a batch with a mask, rounded up to 16 bytes plus
    ceil(L / 32) words per row of the packed mask."""
    import varlen_attention_amd as va
    for B, H, L, bq, bk in ((32, 8, 1584, 128, 128), (3, 5, 100, 32, 64), (1, 1, 1, 64, 32)):
        G = -(-L // 128)
        Tq, Tk = -(-L // bq), -(-L // bk)
        slots = 8 * (-(-(B * H) // 8)) * G
        base = 16 * 3 * slots + 4 * B * G * (Tk + 1) + 4 * B * G * (Tq + 1)
        assert lib.sigattn_schedule_bytes(B, H, L, bq, bk, 0) == base
        assert lib.sigattn_schedule_bytes(B, H, L, bq, bk, 1) == \
            -(-base // 16) * 16 + 4 * B * L * -(-L // 32)
        assert va.schedule_bytes(B, H, L, bq, bk) == base
        assert va.schedule_bytes(B, H, L, bq, bk, dense_mask=True) == \
            lib.sigattn_schedule_bytes(B, H, L, bq, bk, 1)
    assert lib.sigattn_schedule_bytes(0, 1, 10, 32, 32, 0) == va.ERR_INVALID_ARG
    assert lib.sigattn_schedule_bytes(1, 1, 10, 48, 32, 0) == va.ERR_UNSUPPORTED


def test_binding_rejects_cpu_tensors():
    import torch

    import varlen_attention_amd as va
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        va.sigattn_fwd(q, q, q, torch.zeros(1, dtype=torch.int32))


def test_max_masked_length_matches_header():
    """The binding's MAX_MASKED_L is the header's SIGATTN_MAX_MASKED_L."""
    import varlen_attention_amd as va
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "sigattn.h")).read()
    m = re.search(r"#define\s+SIGATTN_MAX_MASKED_L\s+(\d+)", hdr)
    assert m and int(m.group(1)) == va.MAX_MASKED_L



def test_error_messages_are_per_thread(lib):
    """sigattn_last_error is thread-local: two host threads failing for
    different reasons at the same time each read back their own message."""
    import threading

    import varlen_attention_amd as va
    bad = {"head dim": _shape(va, d=96), "must be positive": _shape(va, B=0)}
    errors = []

    def worker(expect, shape):
        for _ in range(2000):
            st = _fwd(lib, va, shape)
            msg = lib.sigattn_last_error().decode()
            if st == va.OK or expect not in msg:
                errors.append((expect, st, msg))
                return

    threads = [threading.Thread(target=worker, args=item) for item in bad.items()]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
