"""Python binding of libdiffattn, the gfx950 differential-attention forward library.

Argument marshalling only: every step of the computation runs in the HIP kernels behind the
C ABI declared in ``include/diffattn.h``.  PyTorch supplies device memory and the stream; the
binding checks that the tensors' shapes agree with each other (the C ABI sees raw pointers and
cannot), builds the strided tensor descriptors and raises ``DiffAttnError`` on any non-OK
status.  There is no fallback: if the shared library is missing or the tensors are not on a
GPU, the call fails.

Entry points (same names as the C ABI):
  diffattn_fwd_v1(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, layer, ...)   V1 prefill
  diffattn_fwd_v2(q1, q2, k, v, lq1, lk1, lq2, lk2, layer, ...)        V2 prefill (GQA pairs)
  (both take window=W for the causal sliding window: diffattn_fwd_v1_window / _v2_window)
  diffattn_fwd_v2_workspace_bytes(B, Hkv, N, D)
  diffattn_decode(q1, q2, kcache, vcache, lq1, lk1, lq2, lk2, layer, ...)  V2 decode step
  diffattn_decode_workspace_bytes(B, P, Hkv, L, D, num_splits=0)
  diffattn_decode_noalloc(q1, q2, kcache, vcache, lq1, ...)   V2 decode step without a workspace
      (its partials use the library's fixed per-GPU scratch)
  diffattn_decode_paged(q1, q2, k_pages, v_pages, block_table, seq_lens, lq1, ...)  V2 decode,
      paged KV cache with per-sequence lengths
  diffattn_decode_v1(q1, q2, k1cache, k2cache, vcache, lq1, lk1, lq2, lk2, layer, ...)  V1 decode
  diffattn_decode_v1_workspace_bytes(B, H, L, d, num_splits=0)
  diffattn_fwd_v1_train(...), diffattn_bwd_v1(...)   V1 training forward (with stash) and backward
  diffattn_lambda_init(layer)
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "DiffAttnError", "load_library", "LIB_PATH",
    "DA_F32", "DA_BF16", "DA_V1_NO_NORM",
    "diffattn_fwd_v1", "diffattn_fwd_v2", "diffattn_decode", "diffattn_decode_noalloc",
    "diffattn_decode_v1", "DIFFATTN_DECODE_NOALLOC_MAX_BYTES",
    "diffattn_decode_paged", "diffattn_fwd_v1_train", "diffattn_bwd_v1",
    "diffattn_v1_train_stash_bytes", "diffattn_bwd_v1_workspace_bytes",
    "diffattn_fwd_v2_workspace_bytes", "diffattn_decode_workspace_bytes",
    "diffattn_decode_v1_workspace_bytes", "diffattn_lambda_init",
    "diffattn_status_string", "diffattn_version",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdiffattn.so")

DA_F32 = 0
DA_BF16 = 1
DA_V1_NO_NORM = 1
DIFFATTN_DECODE_NOALLOC_MAX_BYTES = 16 << 20   # the fixed scratch of diffattn_decode_noalloc

STATUS_NAMES = {0: "DA_OK", 1: "DA_ERR_NULL", 2: "DA_ERR_SHAPE", 3: "DA_ERR_UNSUPPORTED",
                4: "DA_ERR_WORKSPACE", 5: "DA_ERR_HIP"}


class DaTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64),
                ("sn", ctypes.c_int64)]


class DaLambda(ctypes.Structure):
    _fields_ = [("lq1", ctypes.c_void_p), ("lk1", ctypes.c_void_p), ("lq2", ctypes.c_void_p),
                ("lk2", ctypes.c_void_p), ("dl", ctypes.c_int32), ("layer", ctypes.c_int32),
                ("lambda_override", ctypes.c_void_p), ("lambda_out", ctypes.c_void_p)]


class DaLambdaGrad(ctypes.Structure):
    _fields_ = [("dlq1", ctypes.c_void_p), ("dlk1", ctypes.c_void_p), ("dlq2", ctypes.c_void_p),
                ("dlk2", ctypes.c_void_p)]


class DiffAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} "
                         f"({diffattn_status_string(status)})")


_LIB = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libdiffattn.so (built by ``__graft_entry__.build()``) and declare its signatures."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} is missing: build it first (python __graft_entry__.py build)")
    lib = ctypes.CDLL(p)
    T, L = DaTensor, ctypes.POINTER(DaLambda)
    i32, u32, f32, vp, sz = ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    lib.diffattn_fwd_v1.argtypes = [T, T, T, T, T, T, i32, i32, i32, i32, i32, L, i32, f32, u32, vp]
    lib.diffattn_fwd_v1.restype = i32
    lib.diffattn_fwd_v2_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.diffattn_fwd_v2_workspace_bytes.restype = sz
    lib.diffattn_fwd_v2.argtypes = [T, T, T, T, T, i32, i32, i32, i32, i32, i32, L, i32, vp, sz, vp]
    lib.diffattn_fwd_v2.restype = i32
    lib.diffattn_fwd_v1_window.argtypes = [T, T, T, T, T, T, i32, i32, i32, i32, i32, L, i32, f32, u32, vp]
    lib.diffattn_fwd_v1_window.restype = i32
    lib.diffattn_fwd_v2_window.argtypes = [T, T, T, T, T, i32, i32, i32, i32, i32, i32, L, i32, vp, sz, vp]
    lib.diffattn_fwd_v2_window.restype = i32
    lib.diffattn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.diffattn_decode_workspace_bytes.restype = sz
    lib.diffattn_decode.argtypes = [T, T, T, T, T, i32, i32, i32, i32, i32, i32, L, i32, vp, sz, vp]
    lib.diffattn_decode.restype = i32
    lib.diffattn_decode_noalloc.argtypes = [T, T, T, T, T, i32, i32, i32, i32, i32, i32, L, i32, vp]
    lib.diffattn_decode_noalloc.restype = i32
    lib.diffattn_decode_paged.argtypes = [T, T, vp, vp, vp, vp, T, i32, i32, i32, i32, i32, i32, i32,
                                          i32, i32, L, i32, vp, sz, vp]
    lib.diffattn_decode_paged.restype = i32
    lib.diffattn_v1_train_stash_bytes.argtypes = [i32, i32, i32, i32]
    lib.diffattn_v1_train_stash_bytes.restype = sz
    lib.diffattn_bwd_v1_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.diffattn_bwd_v1_workspace_bytes.restype = sz
    lib.diffattn_fwd_v1_train.argtypes = [T, T, T, T, T, T, i32, i32, i32, i32, i32, L, i32, i32, f32, vp,
                                          sz, vp]
    lib.diffattn_fwd_v1_train.restype = i32
    lib.diffattn_bwd_v1.argtypes = [T, T, T, T, T, T, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, L,
                                    ctypes.POINTER(DaLambdaGrad), i32, i32, f32, vp, sz, vp, sz, vp]
    lib.diffattn_bwd_v1.restype = i32
    lib.diffattn_decode_v1_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.diffattn_decode_v1_workspace_bytes.restype = sz
    lib.diffattn_decode_v1.argtypes = [T, T, T, T, T, T, i32, i32, i32, i32, i32, L, f32, u32, i32,
                                       vp, sz, vp]
    lib.diffattn_decode_v1.restype = i32
    lib.diffattn_lambda_init.argtypes = [i32]
    lib.diffattn_lambda_init.restype = ctypes.c_double
    lib.diffattn_status_string.argtypes = [i32]
    lib.diffattn_status_string.restype = ctypes.c_char_p
    lib.diffattn_version.argtypes = []
    lib.diffattn_version.restype = ctypes.c_char_p
    if path is None:
        _LIB = lib
    return lib


def diffattn_status_string(status: int) -> str:
    return load_library().diffattn_status_string(int(status)).decode()


def diffattn_version() -> str:
    return load_library().diffattn_version().decode()


def diffattn_lambda_init(layer: int) -> float:
    return float(load_library().diffattn_lambda_init(int(layer)))


def diffattn_fwd_v2_workspace_bytes(B, Hkv, N, D) -> int:
    return int(load_library().diffattn_fwd_v2_workspace_bytes(B, Hkv, N, D))


def diffattn_decode_workspace_bytes(B, P, Hkv, L, D, num_splits: int = 0) -> int:
    return int(load_library().diffattn_decode_workspace_bytes(B, P, Hkv, L, D, num_splits))


def diffattn_decode_v1_workspace_bytes(B, H, L, d, num_splits: int = 0) -> int:
    return int(load_library().diffattn_decode_v1_workspace_bytes(B, H, L, d, num_splits))


# ------------------------------------------------------------------------------------------------
# marshalling helpers
# ------------------------------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DA_BF16
    if t.dtype == torch.float32:
        return DA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _desc(t, name, shape) -> DaTensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: last dimension must be contiguous")
    if len(shape) == 4:
        sb, sh, sn = t.stride(0), t.stride(1), t.stride(2)
    else:
        sb, sh, sn = t.stride(0), t.stride(1), 0
    return DaTensor(t.data_ptr(), sb, sh, sn)


def _lambda(lq1, lk1, lq2, lk2, layer, n, override, out, device) -> DaLambda:
    torch = _torch()
    lam = DaLambda()
    lam.layer = int(layer)
    if override is not None:
        if override.dtype != torch.float32 or tuple(override.shape) != (n,) or not override.is_cuda:
            raise ValueError(f"lambda_override must be a float32 GPU tensor of shape ({n},)")
        lam.lambda_override = override.data_ptr()
    else:
        vecs = (lq1, lk1, lq2, lk2)
        if any(x is None for x in vecs):
            raise ValueError("the four lambda vectors are required without lambda_override")
        dl = lq1.shape[-1]
        for nm, x in zip(("lq1", "lk1", "lq2", "lk2"), vecs):
            if x.dtype != torch.float32 or tuple(x.shape) != (n, dl) or not x.is_contiguous() \
                    or not x.is_cuda:
                raise ValueError(f"{nm} must be a contiguous float32 GPU tensor of shape ({n}, {dl})")
        lam.lq1, lam.lk1, lam.lq2, lam.lk2 = (x.data_ptr() for x in vecs)
        lam.dl = int(dl)
    if out is not None:
        if out.dtype != torch.float32 or tuple(out.shape) != (n,) or not out.is_cuda:
            raise ValueError(f"lambda_out must be a float32 GPU tensor of shape ({n},)")
        lam.lambda_out = out.data_ptr()
    return lam


def _stream(device, stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(status, where):
    if status != 0:
        raise DiffAttnError(int(status), where)


# ------------------------------------------------------------------------------------------------
# entry points
# ------------------------------------------------------------------------------------------------

def diffattn_fwd_v1(q1, q2, k1, k2, v, lq1=None, lk1=None, lq2=None, lk2=None, layer=1, *,
                    out=None, causal=True, eps=1e-5, flags=0, window=0, lambda_override=None,
                    lambda_out=None, stream=None):
    """V1 differential attention; q1, q2, k1, k2 [B, H, N, d], v [B, H, N, 2d] -> out [B, H, N, 2d].

    bf16 tensors run the fused MFMA kernel, float32 tensors the fp32 kernel.  Lambda vectors are
    float32 [H, d'] GPU tensors; ``layer`` is the 1-based layer of lambda_init.  ``window`` > 0
    selects the causal sliding window (``diffattn_fwd_v1_window``).
    """
    torch = _torch()
    B, H, N, d = q1.shape
    if out is None:
        out = torch.empty((B, H, N, v.shape[-1]), dtype=q1.dtype, device=q1.device)
    dt = _dtype_code(q1)
    for nm, t in (("q2", q2), ("k1", k1), ("k2", k2), ("v", v), ("out", out)):
        if t.dtype != q1.dtype:
            raise TypeError(f"{nm} dtype {t.dtype} differs from q1 dtype {q1.dtype}")
    descs = [_desc(q1, "q1", (B, H, N, d)), _desc(q2, "q2", (B, H, N, d)),
             _desc(k1, "k1", (B, H, N, d)), _desc(k2, "k2", (B, H, N, d)),
             _desc(v, "v", (B, H, N, 2 * d)), _desc(out, "out", (B, H, N, 2 * d))]
    lam = _lambda(lq1, lk1, lq2, lk2, layer, H, lambda_override, lambda_out, q1.device)
    with torch.cuda.device(q1.device):
        st = _stream(q1.device, stream)
        if window:
            if not causal:
                raise ValueError("the sliding window is a causal one")
            _check(load_library().diffattn_fwd_v1_window(*descs, B, H, N, d, dt, ctypes.byref(lam),
                                                         int(window), float(eps), int(flags), st),
                   "diffattn_fwd_v1_window")
        else:
            _check(load_library().diffattn_fwd_v1(*descs, B, H, N, d, dt, ctypes.byref(lam),
                                                  1 if causal else 0, float(eps), int(flags), st),
                   "diffattn_fwd_v1")
    return out


def diffattn_fwd_v2(q1, q2, k, v, lq1=None, lk1=None, lq2=None, lk2=None, layer=1, *,
                    out=None, causal=True, window=0, lambda_override=None, lambda_out=None,
                    workspace=None, stream=None):
    """V2 differential attention; q1, q2 [B, P, N, D] (query heads 2p and 2p+1), k, v [B, Hkv, N, D]
    -> out [B, P, N, D].  Pair p reads KV head p * Hkv // P.  ``window`` > 0 selects the causal
    sliding window (``diffattn_fwd_v2_window``).  ``workspace``: a device uint8 tensor of at least
    ``diffattn_fwd_v2_workspace_bytes(B, Hkv, N, D)`` bytes (allocated here when None)."""
    torch = _torch()
    B, P, N, D = q1.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty((B, P, N, D), dtype=q1.dtype, device=q1.device)
    dt = _dtype_code(q1)
    for nm, t in (("q2", q2), ("k", k), ("v", v), ("out", out)):
        if t.dtype != q1.dtype:
            raise TypeError(f"{nm} dtype {t.dtype} differs from q1 dtype {q1.dtype}")
    descs = [_desc(q1, "q1", (B, P, N, D)), _desc(q2, "q2", (B, P, N, D)),
             _desc(k, "k", (B, Hkv, N, D)), _desc(v, "v", (B, Hkv, N, D)),
             _desc(out, "out", (B, P, N, D))]
    lam = _lambda(lq1, lk1, lq2, lk2, layer, P, lambda_override, lambda_out, q1.device)
    if window and not causal:
        raise ValueError("the sliding window is a causal one")
    if workspace is None:
        workspace = torch.empty(max(16, diffattn_fwd_v2_workspace_bytes(B, Hkv, N, D)), dtype=torch.uint8,
                                device=q1.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(q1.device):
        st = _stream(q1.device, stream)
        if window:
            _check(load_library().diffattn_fwd_v2_window(*descs, B, P, Hkv, N, D, dt,
                                                         ctypes.byref(lam), int(window), ws, ws_bytes, st),
                   "diffattn_fwd_v2_window")
        else:
            _check(load_library().diffattn_fwd_v2(*descs, B, P, Hkv, N, D, dt, ctypes.byref(lam),
                                                  1 if causal else 0, ws, ws_bytes, st), "diffattn_fwd_v2")
    return out


def diffattn_decode(q1, q2, kcache, vcache, lq1=None, lk1=None, lq2=None, lk2=None, layer=1, *,
                    out=None, num_splits=0, workspace=None, lambda_override=None,
                    lambda_out=None, stream=None):
    """One V2 decode step; q1, q2 [B, P, D], kcache, vcache [B, Hkv, L, D] -> out [B, P, D].

    ``workspace`` is a GPU byte tensor of at least ``diffattn_decode_workspace_bytes`` bytes;
    one is allocated when omitted.
    """
    torch = _torch()
    B, P, D = q1.shape
    Hkv, L = kcache.shape[1], kcache.shape[2]
    if out is None:
        out = torch.empty((B, P, D), dtype=q1.dtype, device=q1.device)
    dt = _dtype_code(q1)
    for nm, t in (("q2", q2), ("kcache", kcache), ("vcache", vcache), ("out", out)):
        if t.dtype != q1.dtype:
            raise TypeError(f"{nm} dtype {t.dtype} differs from q1 dtype {q1.dtype}")
    descs = [_desc(q1, "q1", (B, P, D)), _desc(q2, "q2", (B, P, D)),
             _desc(kcache, "kcache", (B, Hkv, L, D)), _desc(vcache, "vcache", (B, Hkv, L, D)),
             _desc(out, "out", (B, P, D))]
    need = diffattn_decode_workspace_bytes(B, P, Hkv, L, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    lam = _lambda(lq1, lk1, lq2, lk2, layer, P, lambda_override, lambda_out, q1.device)
    with torch.cuda.device(q1.device):
        st = _stream(q1.device, stream)
        _check(load_library().diffattn_decode(*descs, B, P, Hkv, L, D, dt, ctypes.byref(lam),
                                              int(num_splits), workspace.data_ptr(), ws_bytes, st),
               "diffattn_decode")
    return out


def diffattn_decode_noalloc(q1, q2, kcache, vcache, lq1=None, lk1=None, lq2=None, lk2=None,
                            layer=1, *, out, num_splits=0, lambda_override=None, lambda_out=None,
                            stream=None):
    """``diffattn_decode`` without a workspace and without allocating: the caller passes ``out``
    [B, P, D] (and every input); the split partials use the library's fixed per-GPU scratch of
    DIFFATTN_DECODE_NOALLOC_MAX_BYTES.  Calls that overlap on one GPU share that scratch and must
    be ordered."""
    B, P, D = q1.shape
    Hkv, L = kcache.shape[1], kcache.shape[2]
    dt = _dtype_code(q1)
    for nm, t in (("q2", q2), ("kcache", kcache), ("vcache", vcache), ("out", out)):
        if t.dtype != q1.dtype:
            raise TypeError(f"{nm} dtype {t.dtype} differs from q1 dtype {q1.dtype}")
    descs = [_desc(q1, "q1", (B, P, D)), _desc(q2, "q2", (B, P, D)),
             _desc(kcache, "kcache", (B, Hkv, L, D)), _desc(vcache, "vcache", (B, Hkv, L, D)),
             _desc(out, "out", (B, P, D))]
    lam = _lambda(lq1, lk1, lq2, lk2, layer, P, lambda_override, lambda_out, q1.device)
    torch = _torch()
    with torch.cuda.device(q1.device):
        st = _stream(q1.device, stream)
        _check(load_library().diffattn_decode_noalloc(*descs, B, P, Hkv, L, D, dt, ctypes.byref(lam),
                                                      int(num_splits), st),
               "diffattn_decode_noalloc")
    return out


def diffattn_decode_v1(q1, q2, k1cache, k2cache, vcache, lq1=None, lk1=None, lq2=None, lk2=None,
                       layer=1, *, out=None, eps=1e-5, flags=0, num_splits=0, workspace=None,
                       lambda_override=None, lambda_out=None, stream=None):
    """One V1 decode step; q1, q2 [B, H, d], k1cache, k2cache [B, H, L, d], vcache [B, H, L, 2d]
    -> out [B, H, 2d] (RMS-normalised and scaled by 1 - lambda_init unless DA_V1_NO_NORM).

    ``workspace`` is a GPU byte tensor of at least ``diffattn_decode_v1_workspace_bytes`` bytes;
    one is allocated when omitted.
    """
    torch = _torch()
    B, H, d = q1.shape
    L = k1cache.shape[2]
    if out is None:
        out = torch.empty((B, H, vcache.shape[-1]), dtype=q1.dtype, device=q1.device)
    dt = _dtype_code(q1)
    for nm, t in (("q2", q2), ("k1cache", k1cache), ("k2cache", k2cache), ("vcache", vcache),
                  ("out", out)):
        if t.dtype != q1.dtype:
            raise TypeError(f"{nm} dtype {t.dtype} differs from q1 dtype {q1.dtype}")
    descs = [_desc(q1, "q1", (B, H, d)), _desc(q2, "q2", (B, H, d)),
             _desc(k1cache, "k1cache", (B, H, L, d)), _desc(k2cache, "k2cache", (B, H, L, d)),
             _desc(vcache, "vcache", (B, H, L, 2 * d)), _desc(out, "out", (B, H, 2 * d))]
    need = diffattn_decode_v1_workspace_bytes(B, H, L, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    lam = _lambda(lq1, lk1, lq2, lk2, layer, H, lambda_override, lambda_out, q1.device)
    with torch.cuda.device(q1.device):
        st = _stream(q1.device, stream)
        _check(load_library().diffattn_decode_v1(*descs, B, H, L, d, dt, ctypes.byref(lam),
                                                 float(eps), int(flags), int(num_splits),
                                                 workspace.data_ptr(), ws_bytes, st),
               "diffattn_decode_v1")
    return out


def diffattn_decode_paged(q1, q2, k_pages, v_pages, block_table, seq_lens, lq1=None, lk1=None,
                          lq2=None, lk2=None, layer=1, *, max_len=None, out=None, num_splits=0,
                          workspace=None, lambda_override=None, lambda_out=None, stream=None):
    """One V2 decode step on a paged KV cache; q1, q2 [B, P, D]; k_pages, v_pages
    [num_pages, Hkv, page_size, D] (contiguous); block_table int32 [B, max_blocks]; seq_lens
    int32 [B] -> out [B, P, D].  ``max_len`` bounds seq_lens (default max_blocks * page_size)."""
    torch = _torch()
    B, P, D = q1.shape
    num_pages, Hkv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    max_blocks = block_table.shape[1]
    if max_len is None:
        max_len = max_blocks * page_size
    if out is None:
        out = torch.empty((B, P, D), dtype=q1.dtype, device=q1.device)
    dt = _dtype_code(q1)
    for nm, x in (("q2", q2), ("k_pages", k_pages), ("v_pages", v_pages), ("out", out)):
        if x.dtype != q1.dtype:
            raise TypeError(f"{nm} dtype {x.dtype} differs from q1 dtype {q1.dtype}")
    for nm, x, shape in (("k_pages", k_pages, (num_pages, Hkv, page_size, D)),
                         ("v_pages", v_pages, (num_pages, Hkv, page_size, D))):
        if tuple(x.shape) != shape or not x.is_contiguous() or not x.is_cuda:
            raise ValueError(f"{nm} must be a contiguous GPU tensor of shape {shape}")
    for nm, x, shape in (("block_table", block_table, (B, max_blocks)), ("seq_lens", seq_lens, (B,))):
        if x.dtype != torch.int32 or tuple(x.shape) != shape or not x.is_contiguous() or not x.is_cuda:
            raise ValueError(f"{nm} must be a contiguous int32 GPU tensor of shape {shape}")
    descs = [_desc(q1, "q1", (B, P, D)), _desc(q2, "q2", (B, P, D))]
    need = diffattn_decode_workspace_bytes(B, P, Hkv, max_len, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    lam = _lambda(lq1, lk1, lq2, lk2, layer, P, lambda_override, lambda_out, q1.device)
    with torch.cuda.device(q1.device):
        st = _stream(q1.device, stream)
        _check(load_library().diffattn_decode_paged(
            *descs, k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
            seq_lens.data_ptr(), _desc(out, "out", (B, P, D)), B, P, Hkv, D, page_size, num_pages,
            max_blocks, int(max_len), dt, ctypes.byref(lam), int(num_splits), workspace.data_ptr(),
            ws_bytes, st), "diffattn_decode_paged")
    return out


def diffattn_v1_train_stash_bytes(B, H, N, d) -> int:
    return int(load_library().diffattn_v1_train_stash_bytes(B, H, N, d))


def diffattn_bwd_v1_workspace_bytes(B, H, N, d) -> int:
    return int(load_library().diffattn_bwd_v1_workspace_bytes(B, H, N, d))


def diffattn_fwd_v1_train(q1, q2, k1, k2, v, lq1=None, lk1=None, lq2=None, lk2=None, layer=1, *,
                          out=None, causal=True, window=0, eps=1e-5, stash=None,
                          lambda_override=None, lambda_out=None, stream=None):
    """V1 forward (bf16) that also fills the stash the backward pass reads; returns (out, stash).
    ``stash`` is a GPU byte tensor of at least ``diffattn_v1_train_stash_bytes`` bytes."""
    torch = _torch()
    B, H, N, d = q1.shape
    if out is None:
        out = torch.empty((B, H, N, v.shape[-1]), dtype=q1.dtype, device=q1.device)
    need = diffattn_v1_train_stash_bytes(B, H, N, d)
    if stash is None:
        stash = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    if not stash.is_cuda or not stash.is_contiguous():
        raise ValueError("stash must be a contiguous GPU tensor")
    dt = _dtype_code(q1)
    descs = [_desc(q1, "q1", (B, H, N, d)), _desc(q2, "q2", (B, H, N, d)),
             _desc(k1, "k1", (B, H, N, d)), _desc(k2, "k2", (B, H, N, d)),
             _desc(v, "v", (B, H, N, 2 * d)), _desc(out, "out", (B, H, N, 2 * d))]
    lam = _lambda(lq1, lk1, lq2, lk2, layer, H, lambda_override, lambda_out, q1.device)
    with torch.cuda.device(q1.device):
        st = _stream(q1.device, stream)
        _check(load_library().diffattn_fwd_v1_train(
            *descs, B, H, N, d, dt, ctypes.byref(lam), 1 if causal else 0, int(window), float(eps),
            stash.data_ptr(), stash.numel() * stash.element_size(), st), "diffattn_fwd_v1_train")
    return out, stash


def diffattn_bwd_v1(q1, q2, k1, k2, v, dy, lq1=None, lk1=None, lq2=None, lk2=None, layer=1, *,
                    stash, causal=True, window=0, eps=1e-5, workspace=None, grads=None,
                    lambda_override=None, stream=None):
    """Gradients of the V1 output for upstream gradient dy [B, H, N, 2d] (bf16).  Returns a dict
    of fp32 GPU tensors: dq1, dq2, dk1, dk2 [B, H, N, d], dv [B, H, N, 2d] and (unless
    ``lambda_override`` is given) dlq1, dlk1, dlq2, dlk2 [H, dl]."""
    torch = _torch()
    B, H, N, d = q1.shape
    dev = q1.device
    dl = lq1.shape[-1] if lq1 is not None else 1
    if grads is None:
        grads = {k: torch.empty((B, H, N, d), dtype=torch.float32, device=dev) for k in ("dq1", "dq2", "dk1", "dk2")}
        grads["dv"] = torch.empty((B, H, N, 2 * d), dtype=torch.float32, device=dev)
        if lambda_override is None:
            for k in ("dlq1", "dlk1", "dlq2", "dlk2"):
                grads[k] = torch.empty((H, dl), dtype=torch.float32, device=dev)
    for k, shape in (("dq1", (B, H, N, d)), ("dq2", (B, H, N, d)), ("dk1", (B, H, N, d)),
                     ("dk2", (B, H, N, d)), ("dv", (B, H, N, 2 * d))):
        x = grads[k]
        if x.dtype != torch.float32 or tuple(x.shape) != shape or not x.is_contiguous() or not x.is_cuda:
            raise ValueError(f"{k} must be a contiguous float32 GPU tensor of shape {shape}")
    need = diffattn_bwd_v1_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    dt = _dtype_code(q1)
    descs = [_desc(q1, "q1", (B, H, N, d)), _desc(q2, "q2", (B, H, N, d)),
             _desc(k1, "k1", (B, H, N, d)), _desc(k2, "k2", (B, H, N, d)),
             _desc(v, "v", (B, H, N, 2 * d)), _desc(dy, "dy", (B, H, N, 2 * d))]
    lam = _lambda(lq1, lk1, lq2, lk2, layer, H, lambda_override, None, dev)
    lg = DaLambdaGrad()
    if lambda_override is None:
        lg.dlq1, lg.dlk1, lg.dlq2, lg.dlk2 = (grads[k].data_ptr() for k in ("dlq1", "dlk1", "dlq2", "dlk2"))
    with torch.cuda.device(dev):
        st = _stream(dev, stream)
        _check(load_library().diffattn_bwd_v1(
            *descs, *(grads[k].data_ptr() for k in ("dq1", "dq2", "dk1", "dk2", "dv")),
            B, H, N, d, dt, ctypes.byref(lam), ctypes.byref(lg), 1 if causal else 0, int(window),
            float(eps),
            stash.data_ptr(), stash.numel() * stash.element_size(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), st), "diffattn_bwd_v1")
    return grads
