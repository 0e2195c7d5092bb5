"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects
bad arguments with the documented status before touching the device.

No call here passes a complete set of valid arguments, so nothing is ever launched.
"""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_forward_amd as fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fa.h")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_SCALE = (
    0, -1, -2, -3, -4, -5, -6, -7)
FA_ERR_SCRATCH = -8

needs_lib = pytest.mark.skipif(not os.path.exists(fa.LIB_PATH), reason="libfa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("fa_forward", "fa_backward", "fa_backward_workspace_bytes", "fa_status_string", "fa_version"):
        assert required in names


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in fa.h but not exported"


@needs_lib
def test_status_strings_and_version():
    lib = fa.library()
    for st in (FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_HIP,
               FA_ERR_SCALE, FA_ERR_SCRATCH):
        s = lib.fa_status_string(st).decode()
        assert s and s != "unknown status"
    assert lib.fa_status_string(12345).decode() == "unknown status"
    assert lib.fa_version() >= 100


P = ctypes.c_void_p(0x10000)   # aligned, never dereferenced: every call below fails validation
P2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)
NUL = ctypes.c_void_p(0)


def fwd(q=P, k=P, v=P, o=P2, lse=P2, B=1, H=1, N=16, d=64, scale=0.125, causal=0, dtype=fa.FA_BF16):
    return fa.library().fa_forward(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), causal, dtype, NUL)


def bwd(ptrs=None, ws=P2, wsb=1 << 20, B=1, H=1, N=16, d=64, scale=0.125, dtype=fa.FA_BF16):
    ptrs = ptrs or [P] * 9
    return fa.library().fa_backward(*ptrs, ws, wsb, B, H, N, d, ctypes.c_float(scale), 0, dtype, NUL)


@needs_lib
@pytest.mark.parametrize("which", range(5))
def test_forward_null(which):
    args = [P, P, P, P2, P2]
    args[which] = NUL
    assert fwd(*args, d=96) == FA_ERR_NULL  # null wins over every other error


@needs_lib
def test_forward_shape_and_dtype_errors():
    assert fwd(B=0, d=96) == FA_ERR_SHAPE
    assert fwd(H=-1, d=96) == FA_ERR_SHAPE
    assert fwd(N=0, d=96) == FA_ERR_SHAPE
    assert fwd(d=96) == FA_ERR_UNSUPPORTED
    assert fwd(d=32) == FA_ERR_UNSUPPORTED
    assert fwd(d=64, dtype=7) == FA_ERR_UNSUPPORTED
    assert fwd(N=1 << 23, d=128, scale=-1.0) == FA_ERR_SHAPE       # a head of 2^31 fp32 bytes
    assert fwd(B=1 << 16, H=1 << 14, N=64, scale=-1.0) == FA_ERR_SHAPE


@needs_lib
def test_forward_scale_and_alignment_errors():
    assert fwd(scale=0.0) == FA_ERR_SCALE
    assert fwd(scale=-0.5) == FA_ERR_SCALE
    assert fwd(scale=float("inf")) == FA_ERR_SCALE
    assert fwd(scale=float("nan")) == FA_ERR_SCALE
    for i in range(4):
        args = [P, P, P, P2, ctypes.c_void_p(0x20002)]
        args[i] = MIS
        assert fwd(*args) == FA_ERR_ALIGN
    assert fwd(lse=ctypes.c_void_p(0x20002)) == FA_ERR_ALIGN


@needs_lib
def test_backward_errors():
    lib = fa.library()
    assert lib.fa_backward_workspace_bytes(2, 3, 5, 64) == 2 * 3 * 5 * 8
    assert lib.fa_backward_workspace_bytes(0, 3, 5, 64) == 0
    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = NUL
        assert bwd(ptrs, d=96) == FA_ERR_NULL
    assert bwd(d=96) == FA_ERR_UNSUPPORTED
    assert bwd(N=0) == FA_ERR_SHAPE
    assert bwd(dtype=fa.FA_F32) == FA_ERR_UNSUPPORTED
    assert bwd(scale=0.0) == FA_ERR_SCALE
    ptrs = [P] * 9
    ptrs[6] = MIS
    assert bwd(ptrs) == FA_ERR_ALIGN
    assert bwd(ws=NUL) == FA_ERR_WORKSPACE
    assert bwd(wsb=16 * 8 - 1) == FA_ERR_WORKSPACE
    assert bwd(ws=ctypes.c_void_p(0x20004), wsb=128) == FA_ERR_ALIGN


@needs_lib
def test_python_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_forward(q, q, q)


def fwd_ex(q=P, k=P, v=P, o=P2, lse=P2, B=1, Hq=4, Hkv=2, Nq=16, Nk=16, d=96, scale=0.125, causal=0,
           dtype=fa.FA_BF16):
    # d = 96 by default: a call whose other checks pass still fails (FA_ERR_UNSUPPORTED)
    return fa.library().fa_forward_ex(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, ctypes.c_float(scale), causal, dtype,
                                      NUL)


@needs_lib
def test_forward_ex_grouping_and_length_errors():
    assert fwd_ex() == FA_ERR_UNSUPPORTED                      # the grouping and lengths themselves pass
    assert fwd_ex(Hq=3, Hkv=2) == FA_ERR_SHAPE                 # Hq not a multiple of Hkv
    assert fwd_ex(Hkv=0) == FA_ERR_SHAPE
    assert fwd_ex(Nk=0) == FA_ERR_SHAPE
    assert fwd_ex(Nq=17, Nk=16, causal=1) == FA_ERR_SHAPE      # a causal query row would see no key
    assert fwd_ex(Nq=17, Nk=16, causal=0) == FA_ERR_UNSUPPORTED
    assert fwd_ex(Nq=1, Nk=4096, causal=1) == FA_ERR_UNSUPPORTED
    assert fwd_ex(Nk=1 << 23, d=128, scale=-1.0) == FA_ERR_SHAPE  # a key head of 2^31 fp32 bytes
    assert fwd_ex(k=NUL) == FA_ERR_NULL
    # 8 query heads sharing one key/value head at 2^21 rows, d = 128: each head fits 32-bit
    # offsets (2^30 fp32 bytes) but the packed group the 16-bit forward addresses is 2^32
    # bytes, which would wrap; it is rejected, also through the split and sparse entry points
    big = dict(B=1, Hq=8, Hkv=1, Nq=1 << 21, Nk=1 << 21, d=128)
    assert fwd_ex(**big) == FA_ERR_SHAPE
    assert fwd_ex(**dict(big, Hq=4)) == FA_ERR_SHAPE            # 2^31 bytes: still too large
    assert fwd_ex(**dict(big, Hq=2, scale=-1.0)) == FA_ERR_SCALE  # 2^30 bytes: the size passes
    assert fwd_ex(**dict(big, dtype=fa.FA_F32, scale=-1.0)) == FA_ERR_SCALE  # fp32: one head at a time
    lib = fa.library()
    args = (P, P, P, P2, P2, 1, 8, 1, 1 << 21, 1 << 21, 128, ctypes.c_float(0.125), 0)
    assert lib.fa_forward_split(*args, 2, P2, 1 << 40, fa.FA_BF16, NUL) == FA_ERR_SHAPE
    assert lib.fa_forward_sparse(*args, P, 1, 1, NUL, 0, fa.FA_BF16, NUL) == FA_ERR_SHAPE


@needs_lib
def test_backward_ex_workspace_is_per_query_row():
    lib = fa.library()
    B, Hq, Hkv, Nq, Nk = 2, 8, 2, 48, 80
    need = lib.fa_backward_workspace_bytes(B, Hq, Nq, 64)
    assert need == 8 * B * Hq * Nq
    st = lib.fa_backward_ex(P, P, P, P, P, P2, P2, P2, P2, P2, need - 1, B, Hq, Hkv, Nq, Nk, 64,
                            ctypes.c_float(0.125), 1, fa.FA_BF16, NUL)
    assert st == FA_ERR_WORKSPACE
    st = lib.fa_backward_ex(P, P, P, P, P, P2, P2, P2, P2, P2, need, B, Hq, 3, Nq, Nk, 64,
                            ctypes.c_float(0.125), 1, fa.FA_BF16, NUL)
    assert st == FA_ERR_SHAPE
    st = lib.fa_backward_dq_ex(P, P, P, P, P2, P2, P2, need, B, Hq, Hkv, Nk + 1, Nk, 64,
                               ctypes.c_float(0.125), 1, fa.FA_BF16, NUL)
    assert st == FA_ERR_SHAPE
    st = lib.fa_backward_dkdv_ex(P, P, P, P, P2, P2, P2, need, B, Hq, Hkv, Nq, Nk, 64,
                                 ctypes.c_float(0.125), 0, fa.FA_F32, NUL)
    assert st == FA_ERR_UNSUPPORTED


@needs_lib
def test_split_entry_points_validate_before_launch():
    lib = fa.library()
    assert lib.fa_forward_split_workspace_bytes(2, 8, 1, 128, 4) == 4 * 2 * 8 * 1 * (128 + 3) * 4
    assert lib.fa_forward_split_workspace_bytes(2, 8, 1, 128, 1) == 0
    assert lib.fa_forward_split_workspace_bytes(2, 8, 1, 128, 1025) == 0
    # a decode step (one query row per head) is split; a large grid is not
    assert lib.fa_forward_split_count(8, 32, 8, 1, 8192, 128, 1, fa.FA_BF16) > 1
    assert lib.fa_forward_split_count(2, 16, 16, 8192, 8192, 128, 1, fa.FA_BF16) == 1
    # causal 8 x 4096 x 64 prefill: six splits leave 456 workgroups with tiles to process
    # (seven would leave 488, past 9/10 of the 512 target); without the causal triangle
    # every split works, and four reach the target
    assert lib.fa_forward_split_count(1, 8, 8, 4096, 4096, 64, 1, fa.FA_BF16) == 6
    assert lib.fa_forward_split_count(1, 8, 8, 4096, 4096, 64, 0, fa.FA_BF16) == 4
    # the fp32 single head (4 blocks of 64 rows, 8 key tiles of 32): one tile per split
    assert lib.fa_forward_split_count(1, 1, 1, 256, 256, 64, 0, fa.FA_F32) == 8
    assert lib.fa_forward_split_count(1, 16, 16, 4096, 4096, 64, 1, fa.FA_F32) == 1
    need = lib.fa_forward_split_workspace_bytes(1, 4, 1, 128, 4)
    args = (P, P, P, P2, P2, 1, 4, 2, 1, 512, 128, ctypes.c_float(0.125), 1)
    assert lib.fa_forward_split(*args, 4, P2, need - 1, fa.FA_BF16, NUL) == FA_ERR_WORKSPACE
    assert lib.fa_forward_split(*args, 4, NUL, need, fa.FA_BF16, NUL) == FA_ERR_WORKSPACE
    assert lib.fa_forward_split(*args, 4, MIS, need, fa.FA_BF16, NUL) == FA_ERR_ALIGN
    assert lib.fa_forward_split(*args, 0, P2, need, fa.FA_BF16, NUL) == FA_ERR_SHAPE
    assert lib.fa_forward_split(*args, 4, P2, need - 1, fa.FA_F32, NUL) == FA_ERR_WORKSPACE  # fp32 splits too
    bad = (P, P, P, P2, P2, 1, 4, 3, 1, 512, 128, ctypes.c_float(0.125), 1)
    assert lib.fa_forward_split(*bad, 4, P2, need, fa.FA_BF16, NUL) == FA_ERR_SHAPE


@needs_lib
def test_sparse_entry_points_validate_before_launch():
    lib = fa.library()
    base = (P, P, P, P2, P2, 1, 4, 2, 256, 256, 64, ctypes.c_float(0.125), 1)
    assert lib.fa_forward_sparse(*base, NUL, 1, 1, NUL, 0, fa.FA_BF16, NUL) == FA_ERR_NULL
    assert lib.fa_forward_sparse(*base, P, 3, 1, NUL, 0, fa.FA_BF16, NUL) == FA_ERR_SHAPE   # heads not 1 or Hq
    assert lib.fa_forward_sparse(*base, P, 1, 0, NUL, 0, fa.FA_BF16, NUL) == FA_ERR_SHAPE   # nsplit < 1
    assert lib.fa_forward_sparse(*base, P, 1, 1, NUL, 0, fa.FA_F32, NUL) == FA_ERR_UNSUPPORTED
    assert lib.fa_forward_sparse(*base, P, 4, 2, NUL, 0, fa.FA_BF16, NUL) == FA_ERR_WORKSPACE
    need = lib.fa_backward_workspace_bytes(1, 4, 256, 64)
    bargs = (P, P, P, P, P, P2, P2, P2, P2, P2, need, 1, 4, 2, 256, 256, 64, ctypes.c_float(0.125), 1)
    assert lib.fa_backward_sparse(*bargs, NUL, 1, fa.FA_BF16, NUL) == FA_ERR_NULL
    assert lib.fa_backward_sparse(*bargs, P, 2, fa.FA_BF16, NUL) == FA_ERR_SHAPE
    assert lib.fa_backward_sparse(*bargs, P, 1, fa.FA_F32, NUL) == FA_ERR_UNSUPPORTED


@needs_lib
def test_fp8_entry_points_validate_before_launch():
    lib = fa.library()
    assert lib.fa_fp8_scale_count(2, 3, 300, 64, 0) == 2 * 3 * 3
    assert lib.fa_fp8_scale_count(2, 3, 300, 64, 1) == 2 * 3 * 64
    assert lib.fa_fp8_scale_count(0, 3, 300, 64, 1) == 0
    assert lib.fa_quantize_fp8(NUL, P, P2, 1, 1, 64, 64, 0, fa.FA_BF16, NUL) == FA_ERR_NULL
    assert lib.fa_quantize_fp8(P, P, P2, 1, 1, 64, 96, 0, fa.FA_BF16, NUL) == FA_ERR_UNSUPPORTED
    assert lib.fa_quantize_fp8(P, MIS, P2, 1, 1, 64, 64, 0, fa.FA_BF16, NUL) == FA_ERR_ALIGN
    args = [P, P2, P, P2, P, P2, P2, P2]
    assert lib.fa_forward_fp8(*args, 1, 4, 3, 64, 64, 128, ctypes.c_float(0.1), 0, NUL) == FA_ERR_SHAPE
    assert lib.fa_forward_fp8(*args, 1, 4, 2, 65, 64, 128, ctypes.c_float(0.1), 1, NUL) == FA_ERR_SHAPE
    assert lib.fa_forward_fp8(*args, 1, 4, 2, 64, 64, 96, ctypes.c_float(0.1), 0, NUL) == FA_ERR_UNSUPPORTED
    assert lib.fa_forward_fp8(*args, 1, 4, 2, 64, 64, 128, ctypes.c_float(-1.0), 0, NUL) == FA_ERR_SCALE
    bad = [P, P2, P, P2, P, MIS, P2, P2]
    assert lib.fa_forward_fp8(*bad, 1, 4, 2, 64, 64, 128, ctypes.c_float(0.1), 0, NUL) == FA_ERR_ALIGN
    assert lib.fa_forward_fp8(NUL, *args[1:], 1, 4, 2, 64, 64, 128, ctypes.c_float(0.1), 0, NUL) == FA_ERR_NULL


@needs_lib
def test_noalloc_backward_validates_before_launch():
    """The workspace-free backward: the usual argument errors, and FA_ERR_SCRATCH for a call
    whose 8 bytes per query row exceed the 16 MiB static scratch (2^21 rows), checked
    before any device call."""
    lib = fa.library()
    f = ctypes.c_float(0.125)

    def call(ptrs=None, B=1, Hq=4, Hkv=2, Nq=64, Nk=64, d=64, scale=f, causal=1, dtype=fa.FA_BF16):
        ptrs = ptrs or [P] * 9
        return lib.fa_backward_noalloc(*ptrs, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, NUL)

    for i in range(9):
        ptrs = [P] * 9
        ptrs[i] = NUL
        assert call(ptrs, d=96) == FA_ERR_NULL
    assert call(d=96) == FA_ERR_UNSUPPORTED
    assert call(dtype=fa.FA_F32) == FA_ERR_UNSUPPORTED
    assert call(Hkv=3) == FA_ERR_SHAPE
    assert call(Nq=0) == FA_ERR_SHAPE
    assert call(Nq=65, causal=1) == FA_ERR_SHAPE
    assert call(scale=ctypes.c_float(0.0)) == FA_ERR_SCALE
    ptrs = [P] * 9
    ptrs[7] = MIS
    assert call(ptrs) == FA_ERR_ALIGN
    # 2^21 + 1 query rows: one row over the static scratch
    assert call(B=1, Hq=1, Hkv=1, Nq=(1 << 21) + 1, Nk=(1 << 21) + 1) == FA_ERR_SCRATCH
    assert call(B=2, Hq=16, Hkv=16, Nq=(1 << 16) + 1, Nk=(1 << 16) + 1) == FA_ERR_SCRATCH
    # a wrong argument is reported as such even when the call is also too large
    assert call(B=2, Hq=16, Hkv=16, Nq=(1 << 16) + 1, Nk=(1 << 16) + 1, d=96) == FA_ERR_UNSUPPORTED
    assert lib.fa_status_string(FA_ERR_SCRATCH).decode().startswith("fa_backward_noalloc")
