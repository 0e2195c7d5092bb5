"""Exact tiled attention for AMD Instinct MI355X (gfx950): Python binding of libfa.so.

The work runs in HIP kernels behind a C ABI (``include/fa.h``).  This module only
marshals arguments: it checks that tensors live on the GPU, are contiguous and agree in
shape and dtype, allocates outputs with torch when the caller passes none, and calls the
library on torch's current stream.  There is no other code path: if ``libfa.so`` is
missing, every call raises.

    import torch, exact_tiled_attention_forward_amd as fa
    o, lse = fa.fa_forward(q, k, v, causal=True)              # (B, H, N, d) bf16/fp16/fp32
    dq, dk, dv = fa.fa_backward(q, k, v, o, do, lse, causal=True)

k and v may have fewer heads than q (grouped heads) and another length (cross-attention,
a cached K/V); see ``fa_forward``.
"""

from __future__ import annotations

import ctypes
import functools
import math
import os

import torch  # the HIP runtime torch loads is the one libfa.so binds to (same soname)

__all__ = ["MASK_BLOCK", "fa_forward", "fa_forward_fp8", "fa_quantize_fp8", "fa_forward_split_count", "fa_backward", "fa_backward_dq", "fa_backward_dkdv", "fa_backward_noalloc",
           "fa_backward_workspace_bytes",
           "library", "load_library", "FAError", "FA_F32", "FA_F16", "FA_BF16", "LIB_PATH", "RACECHECK_LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
# the race-check build (same results on a perturbed schedule; see csrc/fa_device.h)
RACECHECK_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_racecheck.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

_lib = None


class FAError(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, status: int, text: str):
        super().__init__(f"fa status {status}: {text}")
        self.status = status


def library() -> ctypes.CDLL:
    """Load libfa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """A build of the library at `path` with its C signatures declared (the release build
    is `library()`; the race-check build is RACECHECK_LIB_PATH)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m exact_tiled_attention_forward_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_forward.restype = i
    lib.fa_backward_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_backward_workspace_bytes.restype = sz
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    lib.fa_backward_dq.restype = i
    lib.fa_backward_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    lib.fa_backward_dkdv.restype = i
    lib.fa_forward_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_forward_ex.restype = i
    lib.fa_backward_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_backward_ex.restype = i
    lib.fa_backward_dq_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_backward_dq_ex.restype = i
    lib.fa_backward_dkdv_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_backward_dkdv_ex.restype = i
    lib.fa_forward_split_count.argtypes = [i, i, i, i, i, i, i, i]
    lib.fa_forward_split_count.restype = i
    lib.fa_forward_split_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_forward_split_workspace_bytes.restype = sz
    lib.fa_forward_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, sz, i, vp]
    lib.fa_forward_split.restype = i
    lib.fa_forward_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, i, vp, sz, i, vp]
    lib.fa_forward_sparse.restype = i
    lib.fa_backward_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, vp, i, i,
                                       vp]
    lib.fa_backward_sparse.restype = i
    lib.fa_fp8_scale_count.argtypes = [i, i, i, i, i]
    lib.fa_fp8_scale_count.restype = sz
    lib.fa_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp]
    lib.fa_quantize_fp8.restype = i
    lib.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_forward_fp8.restype = i
    lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_backward_noalloc.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    return lib


def _check(status: int):
    if status != 0:
        raise FAError(status, library().fa_status_string(status).decode())


def _gpu_tensor(name, t, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return ctypes.c_void_p(t.data_ptr())


def _one_device(fn):
    """Run an entry point with the device of its tensor arguments current, after checking
    that they all live on that one device (a kernel launched on one GPU cannot read another
    GPU's memory, and the no-workspace backward keeps its scratch per device)."""
    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        tensors = [(f"argument {i}", a) for i, a in enumerate(args) if isinstance(a, torch.Tensor)]
        tensors += [(k, a) for k, a in kwargs.items() if isinstance(a, torch.Tensor)]
        gpu = [(name, t) for name, t in tensors if t.device.type == "cuda"]
        if not gpu:
            return fn(*args, **kwargs)  # the tensor checks report the CPU tensors
        dev = gpu[0][1].device
        for name, t in gpu:
            if t.device != dev:
                raise ValueError(f"{name} is on {t.device}, {gpu[0][0]} on {dev}: all tensors must be on one device")
        if dev.index is None or dev.index == torch.cuda.current_device():
            return fn(*args, **kwargs)
        with torch.cuda.device(dev):
            return fn(*args, **kwargs)
    return wrapped


def _stream(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _shapes(q, k):
    """(B, Hq, Hkv, Nq, Nk, d) from q (B, Hq, Nq, d) and k (B, Hkv, Nk, d)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D: (B, H, N, d)")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"k must be (B={B}, H_kv, N_k, d={d}) (got {tuple(k.shape)})")
    return B, Hq, Hkv, Nq, Nk, d


@_one_device
def fa_forward_split_count(q, k, causal=False):
    """The key-range split count the library suggests for these shapes (1: no split)."""
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
    return int(library().fa_forward_split_count(B, Hq, Hkv, Nq, Nk, d, int(bool(causal)),
                                                _DTYPE_CODE.get(q.dtype, -1)))


MASK_BLOCK = 128  # rows and columns of one block of a block-sparse mask


def _block_mask(block_mask, Hq, Nq, Nk):
    """Check a (1 or Hq, ceil(Nq/128), ceil(Nk/128)) uint8 GPU mask; returns (pointer, heads)."""
    nb = ((Nq + MASK_BLOCK - 1) // MASK_BLOCK, (Nk + MASK_BLOCK - 1) // MASK_BLOCK)
    if block_mask.dim() != 3 or tuple(block_mask.shape[1:]) != nb or block_mask.shape[0] not in (1, Hq):
        raise ValueError(f"block_mask must be (1 or {Hq}, {nb[0]}, {nb[1]}) (got {tuple(block_mask.shape)})")
    return _gpu_tensor("block_mask", block_mask, torch.uint8), int(block_mask.shape[0])


@_one_device
def fa_forward(q, k, v, o=None, lse=None, *, scale=None, causal=False, stream=None, split=None, workspace=None,
               block_mask=None):
    """O, lse = attention(q, k, v).

    q (B, Hq, Nq, d); k, v (B, Hkv, Nk, d) with Hq a multiple of Hkv (query head h
    reads key/value head h // (Hq // Hkv)); o like q; lse (B, Hq, Nq) float32.  With
    causal=True the queries are the last Nq positions of the Nk keys.

    ``split``: None lets the library choose (fa_forward_split_count: more than one only
    when the grid is too small to fill the GPU, e.g. a decode step), 1 forces one pass
    over the keys, n > 1 splits each query block's key range in up to n chunks merged
    afterwards.  ``workspace`` (uint8, optional) holds the split partials.

    ``block_mask``: optional uint8 GPU tensor (1 or Hq, ceil(Nq/128), ceil(Nk/128)); a 0
    byte hides a 128 x 128 block (see include/fa.h).
    """
    lib = library()
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    pq = _gpu_tensor("q", q, dt)
    pk = _gpu_tensor("k", k, dt)
    pv = _gpu_tensor("v", v, dt, k.shape)
    po = _gpu_tensor("o", o, dt, q.shape)
    pl = _gpu_tensor("lse", lse, torch.float32, (B, Hq, Nq))
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    ns = fa_forward_split_count(q, k, causal) if split is None else int(split)
    if block_mask is not None:
        pm, mh = _block_mask(block_mask, Hq, Nq, Nk)
        pw, nbytes = ctypes.c_void_p(0), 0
        if ns > 1:
            nbytes = int(lib.fa_forward_split_workspace_bytes(B, Hq, Nq, d, ns))
            if workspace is None:
                workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
            pw, nbytes = _gpu_tensor("workspace", workspace), workspace.numel() * workspace.element_size()
        _check(lib.fa_forward_sparse(pq, pk, pv, po, pl, B, Hq, Hkv, Nq, Nk, d, ctypes.c_float(sc), int(bool(causal)),
                                     pm, mh, max(ns, 1), pw, nbytes, _DTYPE_CODE[dt], _stream(stream, q.device)))
        return o, lse
    if ns > 1:
        need = int(lib.fa_forward_split_workspace_bytes(B, Hq, Nq, d, ns))
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        pw = _gpu_tensor("workspace", workspace)
        _check(lib.fa_forward_split(pq, pk, pv, po, pl, B, Hq, Hkv, Nq, Nk, d, ctypes.c_float(sc),
                                    int(bool(causal)), ns, pw, workspace.numel() * workspace.element_size(),
                                    _DTYPE_CODE[dt], _stream(stream, q.device)))
        return o, lse
    if Hq == Hkv and Nq == Nk:  # the square entry point itself
        _check(lib.fa_forward(pq, pk, pv, po, pl, B, Hq, Nq, d, ctypes.c_float(sc), int(bool(causal)),
                              _DTYPE_CODE[dt], _stream(stream, q.device)))
        return o, lse
    _check(lib.fa_forward_ex(pq, pk, pv, po, pl, B, Hq, Hkv, Nq, Nk, d, ctypes.c_float(sc), int(bool(causal)),
                             _DTYPE_CODE[dt], _stream(stream, q.device)))
    return o, lse


def fa_backward_workspace_bytes(B, H, N, d):
    """Workspace bytes of the backward for B batches, H query heads and N query rows."""
    return int(library().fa_backward_workspace_bytes(B, H, N, d))


def _workspace(q, workspace):
    B, Hq, Nq, d = q.shape
    if workspace is None:
        workspace = torch.empty(max(fa_backward_workspace_bytes(B, Hq, Nq, d), 16), dtype=torch.uint8, device=q.device)
    return workspace


@_one_device
def fa_backward(q, k, v, o, do, lse, dq=None, dk=None, dv=None, *, scale=None, causal=False,
                workspace=None, stream=None, block_mask=None):
    """dQ (like q), dK, dV (like k) as float32 gradients of sum(O * dO), recomputing P from
    q, k and lse.  Shapes, grouping and block_mask as for fa_forward."""
    lib = library()
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
    dt, f32 = q.dtype, torch.float32
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    dq = torch.empty(q.shape, dtype=f32, device=q.device) if dq is None else dq
    dk = torch.empty(k.shape, dtype=f32, device=q.device) if dk is None else dk
    dv = torch.empty(k.shape, dtype=f32, device=q.device) if dv is None else dv
    workspace = _workspace(q, workspace)
    ptrs = [_gpu_tensor("q", q, dt), _gpu_tensor("k", k, dt), _gpu_tensor("v", v, dt, k.shape),
            _gpu_tensor("o", o, dt, q.shape), _gpu_tensor("do", do, dt, q.shape),
            _gpu_tensor("lse", lse, f32, (B, Hq, Nq)), _gpu_tensor("dq", dq, f32, q.shape),
            _gpu_tensor("dk", dk, f32, k.shape), _gpu_tensor("dv", dv, f32, k.shape),
            _gpu_tensor("workspace", workspace)]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if block_mask is not None:
        pm, mh = _block_mask(block_mask, Hq, Nq, Nk)
        _check(lib.fa_backward_sparse(*ptrs, workspace.numel() * workspace.element_size(), B, Hq, Hkv, Nq, Nk, d,
                                      ctypes.c_float(sc), int(bool(causal)), pm, mh, _DTYPE_CODE[dt],
                                      _stream(stream, q.device)))
        return dq, dk, dv
    if Hq == Hkv and Nq == Nk:  # the square entry point itself
        _check(lib.fa_backward(*ptrs, workspace.numel() * workspace.element_size(), B, Hq, Nq, d,
                               ctypes.c_float(sc), int(bool(causal)), _DTYPE_CODE[dt], _stream(stream, q.device)))
        return dq, dk, dv
    _check(lib.fa_backward_ex(*ptrs, workspace.numel() * workspace.element_size(), B, Hq, Hkv, Nq, Nk, d,
                              ctypes.c_float(sc), int(bool(causal)), _DTYPE_CODE[dt], _stream(stream, q.device)))
    return dq, dk, dv


@_one_device
def fa_backward_noalloc(q, k, v, o, do, lse, dq, dk, dv, *, scale=None, causal=False, stream=None):
    """fa_backward without a workspace: the row statistics live in the library's static
    device scratch (at most 2^21 query rows B*Hq*Nq; see include/fa.h).  dq, dk, dv are
    the caller's float32 outputs; nothing is allocated.  Calls that overlap in time on
    one device race on the shared scratch."""
    lib = library()
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
    dt, f32 = q.dtype, torch.float32
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    ptrs = [_gpu_tensor("q", q, dt), _gpu_tensor("k", k, dt), _gpu_tensor("v", v, dt, k.shape),
            _gpu_tensor("o", o, dt, q.shape), _gpu_tensor("do", do, dt, q.shape),
            _gpu_tensor("lse", lse, f32, (B, Hq, Nq)), _gpu_tensor("dq", dq, f32, q.shape),
            _gpu_tensor("dk", dk, f32, k.shape), _gpu_tensor("dv", dv, f32, k.shape)]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib.fa_backward_noalloc(*ptrs, B, Hq, Hkv, Nq, Nk, d, ctypes.c_float(sc), int(bool(causal)),
                                   _DTYPE_CODE[dt], _stream(stream, q.device)))
    return dq, dk, dv


@_one_device
def fa_backward_dq(q, k, v, do, lse, dq=None, *, scale=None, causal=False, workspace=None, stream=None):
    """First backward stage: dQ, plus D and lse*log2(e) in ``workspace`` (returned) for
    fa_backward_dkdv."""
    lib = library()
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
    dt, f32 = q.dtype, torch.float32
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    workspace = _workspace(q, workspace)
    dq = torch.empty(q.shape, dtype=f32, device=q.device) if dq is None else dq
    ptrs = [_gpu_tensor("q", q, dt), _gpu_tensor("k", k, dt), _gpu_tensor("v", v, dt, k.shape),
            _gpu_tensor("do", do, dt, q.shape), _gpu_tensor("lse", lse, f32, (B, Hq, Nq)),
            _gpu_tensor("dq", dq, f32, q.shape), _gpu_tensor("workspace", workspace)]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if Hq == Hkv and Nq == Nk:
        _check(lib.fa_backward_dq(*ptrs, workspace.numel() * workspace.element_size(), B, Hq, Nq, d,
                                  ctypes.c_float(sc), int(bool(causal)), _DTYPE_CODE[dt], _stream(stream, q.device)))
        return dq, workspace
    _check(lib.fa_backward_dq_ex(*ptrs, workspace.numel() * workspace.element_size(), B, Hq, Hkv, Nq, Nk, d,
                                 ctypes.c_float(sc), int(bool(causal)), _DTYPE_CODE[dt], _stream(stream, q.device)))
    return dq, workspace


@_one_device
def fa_backward_dkdv(q, k, v, do, workspace, dk=None, dv=None, *, scale=None, causal=False, stream=None):
    """Second backward stage: dK, dV from the workspace fa_backward_dq filled."""
    lib = library()
    B, Hq, Hkv, Nq, Nk, d = _shapes(q, k)
    dt, f32 = q.dtype, torch.float32
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    if workspace is None:
        raise ValueError("fa_backward_dkdv needs the workspace fa_backward_dq filled")
    dk = torch.empty(k.shape, dtype=f32, device=q.device) if dk is None else dk
    dv = torch.empty(k.shape, dtype=f32, device=q.device) if dv is None else dv
    ptrs = [_gpu_tensor("q", q, dt), _gpu_tensor("k", k, dt), _gpu_tensor("v", v, dt, k.shape),
            _gpu_tensor("do", do, dt, q.shape), _gpu_tensor("dk", dk, f32, k.shape),
            _gpu_tensor("dv", dv, f32, k.shape), _gpu_tensor("workspace", workspace)]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if Hq == Hkv and Nq == Nk:
        _check(lib.fa_backward_dkdv(*ptrs, workspace.numel() * workspace.element_size(), B, Hq, Nq, d,
                                    ctypes.c_float(sc), int(bool(causal)), _DTYPE_CODE[dt], _stream(stream, q.device)))
        return dk, dv
    _check(lib.fa_backward_dkdv_ex(*ptrs, workspace.numel() * workspace.element_size(), B, Hq, Hkv, Nq, Nk, d,
                                   ctypes.c_float(sc), int(bool(causal)), _DTYPE_CODE[dt], _stream(stream, q.device)))
    return dk, dv


@_one_device
def fa_quantize_fp8(x, *, per_channel=False, stream=None):
    """E4M3 codes (uint8, like x) and float32 scales of x (B, H, N, d): one scale per 128
    rows of a head, or per channel of a head with per_channel=True."""
    lib = library()
    if x.dim() != 4:
        raise ValueError("x must be (B, H, N, d)")
    B, H, N, d = x.shape
    if x.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {x.dtype}")
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    shape = (B, H, d) if per_channel else (B, H, (N + 127) // 128)
    scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    _check(lib.fa_quantize_fp8(_gpu_tensor("x", x), _gpu_tensor("codes", codes), _gpu_tensor("scales", scales),
                               B, H, N, d, int(bool(per_channel)), _DTYPE_CODE[x.dtype], _stream(stream, x.device)))
    return codes, scales


@_one_device
def fa_forward_fp8(q8, q_scale, k8, k_scale, v8, v_scale, o=None, lse=None, *, scale=None, causal=False,
                   stream=None):
    """O (bf16, like q8) and lse from E4M3 codes and their scales (see fa_quantize_fp8: row
    blocks for q and k, channels for v)."""
    lib = library()
    B, Hq, Hkv, Nq, Nk, d = _shapes(q8, k8)
    u8, f32 = torch.uint8, torch.float32
    if o is None:
        o = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=f32, device=q8.device)
    ptrs = [_gpu_tensor("q8", q8, u8), _gpu_tensor("q_scale", q_scale, f32, (B, Hq, (Nq + 127) // 128)),
            _gpu_tensor("k8", k8, u8), _gpu_tensor("k_scale", k_scale, f32, (B, Hkv, (Nk + 127) // 128)),
            _gpu_tensor("v8", v8, u8, k8.shape), _gpu_tensor("v_scale", v_scale, f32, (B, Hkv, d)),
            _gpu_tensor("o", o, torch.bfloat16, q8.shape), _gpu_tensor("lse", lse, f32, (B, Hq, Nq))]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _check(lib.fa_forward_fp8(*ptrs, B, Hq, Hkv, Nq, Nk, d, ctypes.c_float(sc), int(bool(causal)),
                              _stream(stream, q8.device)))
    return o, lse
