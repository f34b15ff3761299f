"""Thin Python binding of libfa2.so (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI
declared in ``include/fa2.h``; this module only checks tensor properties,
allocates outputs with PyTorch (device memory and streams are all PyTorch is
used for) and forwards raw pointers.  There is no fallback: if the library is
missing or a call fails, an exception is raised.

Functions mirror the C entry points: ``fwd``, ``bwd``, ``bwd_workspace_bytes``,
``bwd_rows_padded``, ``bwd_preprocess``, ``bwd_dkdv``, ``bwd_dq``, ``tile_config``.
Query and key lengths are taken from the tensors: q, o, do, dq hold Nq rows,
k, v, dk, dv hold Nk rows; with Nq == Nk the plain entry points are called,
otherwise their ``_qk`` variants (causal mask aligned bottom-right).  Tensors
need a contiguous last dimension only: when any bf16 tensor of a call is not
contiguous [B, H, N, d] (a [B, N, H, d] tensor seen through ``transpose(1, 2)``,
a head group of a fused QKV projection), ``fwd`` and ``bwd`` pass element
strides to ``fa2_fwd_strided`` / ``fa2_bwd_strided`` instead of copying.
float16 tensors (all 16-bit tensors of a call share one type) go through the
strided entry points with ``FA2_FP16``.
"""

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa2.so")

FA2_OK = 0
FA2_BF16, FA2_FP16 = 0, 1
SUPPORTED_HEAD_DIMS = (64, 80, 96, 128, 256)

_lib = None

_c_ptr = ctypes.c_void_p
_c_int = ctypes.c_int
_c_float = ctypes.c_float
_c_size = ctypes.c_size_t

class Strides(ctypes.Structure):
    """fa2_strides: element strides of the batch, head and row dimensions."""
    _fields_ = [("batch", ctypes.c_longlong), ("head", ctypes.c_longlong), ("row", ctypes.c_longlong)]


_c_strides = ctypes.POINTER(Strides)

_SIGNATURES = {
    "fa2_fwd_strided": (_c_int, [_c_ptr, _c_strides] * 4 + [_c_ptr] + [_c_int] * 5
                        + [_c_float, _c_int, _c_int, _c_ptr]),
    "fa2_bwd_strided": (_c_int, [_c_ptr, _c_strides] * 4 + [_c_ptr] + [_c_ptr, _c_strides] * 4
                        + [_c_int] * 5 + [_c_float, _c_int, _c_int, _c_ptr, _c_size, _c_ptr]),
    "fa2_fwd": (_c_int, [_c_ptr] * 5 + [_c_int] * 4 + [_c_float, _c_int, _c_ptr]),
    "fa2_fwd_qk": (_c_int, [_c_ptr] * 5 + [_c_int] * 5 + [_c_float, _c_int, _c_ptr]),
    "fa2_bwd_qk": (_c_int, [_c_ptr] * 9 + [_c_int] * 5 + [_c_float, _c_int, _c_ptr, _c_size, _c_ptr]),
    "fa2_bwd_qk_noalloc": (_c_int, [_c_ptr] * 9 + [_c_int] * 5 + [_c_float, _c_int, _c_ptr]),
    "fa2_bwd_noalloc_max_bytes": (_c_size, []),
    "fa2_bwd_dkdv_qk": (_c_int, [_c_ptr] * 8 + [_c_int] * 5 + [_c_float, _c_int, _c_ptr]),
    "fa2_bwd_dq_qk": (_c_int, [_c_ptr] * 7 + [_c_int] * 5 + [_c_float, _c_int, _c_ptr]),
    "fa2_bwd_rows_padded": (_c_int, [_c_int]),
    "fa2_bwd_workspace_bytes": (_c_size, [_c_int] * 4),
    "fa2_bwd": (_c_int, [_c_ptr] * 9 + [_c_int] * 4 + [_c_float, _c_int, _c_ptr, _c_size, _c_ptr]),
    "fa2_bwd_preprocess": (_c_int, [_c_ptr] * 5 + [_c_int] * 4 + [_c_ptr]),
    "fa2_bwd_dkdv": (_c_int, [_c_ptr] * 8 + [_c_int] * 4 + [_c_float, _c_int, _c_ptr]),
    "fa2_bwd_dq": (_c_int, [_c_ptr] * 7 + [_c_int] * 4 + [_c_float, _c_int, _c_ptr]),
    "fa2_strerror": (ctypes.c_char_p, [_c_int]),
    "fa2_last_error": (ctypes.c_char_p, []),
    "fa2_tile_config": (_c_int, [_c_int] + [ctypes.POINTER(_c_int)] * 6),
}


class FA2Error(RuntimeError):
    def __init__(self, status, where):
        lib = load()
        msg = lib.fa2_strerror(status).decode()
        detail = lib.fa2_last_error().decode()
        super().__init__(f"{where}: status {status}: {msg}" + (f" [{detail}]" if detail and status == 4 else ""))
        self.status = status


def load(path=None):
    """Load libfa2.so (built by ``exact_tiled_attention_34_amd.build``).

    With a path, that library is loaded and becomes the one every function of
    this module calls."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build it with `python -m exact_tiled_attention_34_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (restype, argtypes) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = restype
        fn.argtypes = argtypes
    _lib = lib
    return lib


def _check(status, where):
    if status != FA2_OK:
        raise FA2Error(status, where)


def _stream_handle(device, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check_qkv(name, t, shape=None, strided_ok=False):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"{name} must be bfloat16 or float16, got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, N, d]")
    if strided_ok:
        if t.stride(3) != 1:
            raise ValueError(f"{name} needs a contiguous last dimension")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dtype_code(tensors):
    """FA2_BF16 / FA2_FP16 for a call whose 16-bit tensors must share one type."""
    import torch
    kinds = {t.dtype for t in tensors}
    if len(kinds) != 1:
        raise ValueError(f"all 16-bit tensors of a call must share one dtype, got {sorted(map(str, kinds))}")
    return FA2_FP16 if kinds.pop() == torch.float16 else FA2_BF16


def _strides(t):
    """fa2_strides of a [B, H, N, d] tensor (element strides), by reference.  A
    dimension of size 1 is never stepped over, so its stride (which PyTorch may
    report as any value) is passed as 0."""
    return ctypes.byref(Strides(*(t.stride(i) if t.shape[i] > 1 else 0 for i in range(3))))


def _check_f32(name, t, shape):
    import torch
    if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 GPU tensor of shape {tuple(shape)}")


def default_scale(d):
    return 1.0 / math.sqrt(d)


def _key_shape(q, k):
    """[B, H, Nk, d] with Nk taken from k (after checking k itself)."""
    _check_qkv("k", k, strided_ok=True)
    return (q.shape[0], q.shape[1], k.shape[2], q.shape[3])


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None):
    """O, L = attention(q, k, v); q bf16 [B,H,Nq,d], k/v bf16 [B,H,Nk,d] on the GPU.

    Any of q, k, v, out may be a strided view with a contiguous last dimension."""
    import torch
    _check_qkv("q", q, strided_ok=True)
    B, H, N, d = q.shape
    kshape = _key_shape(q, k)
    _check_qkv("k", k, kshape, strided_ok=True)
    _check_qkv("v", v, kshape, strided_ok=True)
    Nk = kshape[2]
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_qkv("out", out, q.shape, strided_ok=True)
    _check_f32("lse", lse, (B, H, N))
    code = _dtype_code((q, k, v, out))
    tail = (scale, int(bool(causal)), _stream_handle(q.device, stream))
    if code == FA2_BF16 and all(t.is_contiguous() for t in (q, k, v, out)):
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
        if Nk == N:
            st = load().fa2_fwd(*ptrs, B, H, N, d, *tail)
        else:
            st = load().fa2_fwd_qk(*ptrs, B, H, N, Nk, d, *tail)
    else:
        st = load().fa2_fwd_strided(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(),
                                    _strides(v), out.data_ptr(), _strides(out), lse.data_ptr(),
                                    B, H, N, Nk, d, scale, int(bool(causal)), code,
                                    _stream_handle(q.device, stream))
    _check(st, "fa2_fwd")
    return out, lse


def bwd_workspace_bytes(B, H, N, d):
    return int(load().fa2_bwd_workspace_bytes(B, H, N, d))


def bwd(q, k, v, o, lse, do, causal=False, scale=None, dq=None, dk=None, dv=None,
        workspace=None, stream=None):
    """dQ, dK, dV of sum(do * o); q/o/do/dq bf16 [B,H,Nq,d], k/v/dk/dv bf16 [B,H,Nk,d], lse fp32 [B,H,Nq]."""
    import torch
    _check_qkv("q", q, strided_ok=True)
    B, H, N, d = q.shape
    kshape = _key_shape(q, k)
    Nk = kshape[2]
    for name, t, shape in (("k", k, kshape), ("v", v, kshape), ("o", o, q.shape), ("do", do, q.shape)):
        _check_qkv(name, t, shape, strided_ok=True)
    _check_f32("lse", lse, (B, H, N))
    scale = default_scale(d) if scale is None else float(scale)
    dq = torch.empty(q.shape, dtype=q.dtype, device=q.device) if dq is None else dq
    dk = torch.empty(kshape, dtype=q.dtype, device=q.device) if dk is None else dk
    dv = torch.empty(kshape, dtype=q.dtype, device=q.device) if dv is None else dv
    for name, t, shape in (("dq", dq, q.shape), ("dk", dk, kshape), ("dv", dv, kshape)):
        _check_qkv(name, t, shape, strided_ok=True)
    need = bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws = (workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream_handle(q.device, stream))
    tail = (scale, int(bool(causal))) + ws
    tensors = (q, k, v, o, do, dq, dk, dv)
    code = _dtype_code(tensors)
    if code == FA2_BF16 and all(t.is_contiguous() for t in tensors):
        ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr())
        if Nk == N:
            st = load().fa2_bwd(*ptrs, B, H, N, d, *tail)
        else:
            st = load().fa2_bwd_qk(*ptrs, B, H, N, Nk, d, *tail)
    else:
        args = []
        for t in (q, k, v, o):
            args += [t.data_ptr(), _strides(t)]
        args.append(lse.data_ptr())
        for t in (do, dq, dk, dv):
            args += [t.data_ptr(), _strides(t)]
        st = load().fa2_bwd_strided(*args, B, H, N, Nk, d, scale, int(bool(causal)), code, *ws)
    _check(st, "fa2_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, causal=False, scale=None, stream=None):
    """fa2_bwd_qk_noalloc: the backward with the library's fixed device scratch instead
    of a workspace.  Contiguous bfloat16 tensors; the caller passes the outputs dq
    [B,H,Nq,d], dk and dv [B,H,Nk,d], so that nothing is allocated.  Calls that
    overlap in time on one GPU share (and race on) its scratch."""
    import torch
    B, H, N, d, Nk, kshape = _phase_shapes(q, k)
    for name, t, shape in (("q", q, q.shape), ("k", k, kshape), ("v", v, kshape), ("o", o, q.shape),
                           ("do", do, q.shape), ("dq", dq, q.shape), ("dk", dk, kshape), ("dv", dv, kshape)):
        _check_qkv(name, t, shape)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name}: fa2_bwd_qk_noalloc takes bfloat16 tensors, got {t.dtype}")
    _check_f32("lse", lse, (B, H, N))
    scale = default_scale(d) if scale is None else float(scale)
    st = load().fa2_bwd_qk_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                   B, H, N, Nk, d, scale, int(bool(causal)), _stream_handle(q.device, stream))
    _check(st, "fa2_bwd_qk_noalloc")
    return dq, dk, dv


def bwd_noalloc_max_bytes():
    return int(load().fa2_bwd_noalloc_max_bytes())


def bwd_rows_padded(N):
    return int(load().fa2_bwd_rows_padded(N))


def bwd_row_arrays(B, H, N, device):
    """Allocate the two padded fp32 row arrays (delta, L*log2 e) of the backward phases."""
    import torch
    shape = (B, H, bwd_rows_padded(N))
    return (torch.empty(shape, dtype=torch.float32, device=device),
            torch.empty(shape, dtype=torch.float32, device=device))


def _check_phase_tensors(named, rows_shape):
    """The phase entry points take contiguous bfloat16 [B,H,N,d] tensors and the two
    padded fp32 row arrays [B,H,bwd_rows_padded(Nq)]: anything else (another dtype,
    a strided or expanded view) is rejected here, before any pointer reaches the C ABI."""
    import torch
    for name, t, shape in named:
        _check_qkv(name, t, shape)
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name}: the phase entry points take bfloat16 tensors, got {t.dtype}")
    for name, t in rows_shape[1]:
        _check_f32(name, t, rows_shape[0])


def bwd_preprocess(o, do, lse, delta, lse_log2, stream=None):
    """delta = rowsum(do * o) and lse_log2 = lse * log2(e) into the padded row arrays."""
    _check_qkv("o", o)
    B, H, N, d = o.shape
    _check_f32("lse", lse, (B, H, N))
    _check_phase_tensors((("o", o, o.shape), ("do", do, o.shape)),
                         ((B, H, bwd_rows_padded(N)), (("delta", delta), ("lse_log2", lse_log2))))
    st = load().fa2_bwd_preprocess(o.data_ptr(), do.data_ptr(), lse.data_ptr(), delta.data_ptr(),
                                   lse_log2.data_ptr(), B, H, N, d, _stream_handle(o.device, stream))
    _check(st, "fa2_bwd_preprocess")


def _phase_shapes(q, k):
    _check_qkv("q", q)
    _check_qkv("k", k)
    B, H, N, d = q.shape
    return B, H, N, d, k.shape[2], (B, H, k.shape[2], d)


def bwd_dkdv(q, k, v, do, lse_log2, delta, dk, dv, causal=False, scale=None, stream=None):
    """dK, dV from the row arrays of bwd_preprocess (contiguous bf16 tensors only)."""
    B, H, N, d, Nk, kshape = _phase_shapes(q, k)
    _check_phase_tensors((("q", q, q.shape), ("k", k, kshape), ("v", v, kshape), ("do", do, q.shape),
                          ("dk", dk, kshape), ("dv", dv, kshape)),
                         ((B, H, bwd_rows_padded(N)), (("lse_log2", lse_log2), ("delta", delta))))
    scale = default_scale(d) if scale is None else float(scale)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
            lse_log2.data_ptr(), delta.data_ptr(), dk.data_ptr(), dv.data_ptr())
    tail = (scale, int(bool(causal)), _stream_handle(q.device, stream))
    if Nk == N:
        st = load().fa2_bwd_dkdv(*ptrs, B, H, N, d, *tail)
    else:
        st = load().fa2_bwd_dkdv_qk(*ptrs, B, H, N, Nk, d, *tail)
    _check(st, "fa2_bwd_dkdv")


def bwd_dq(q, k, v, do, lse_log2, delta, dq, causal=False, scale=None, stream=None):
    """dQ from the row arrays of bwd_preprocess (contiguous bf16 tensors only)."""
    B, H, N, d, Nk, kshape = _phase_shapes(q, k)
    _check_phase_tensors((("q", q, q.shape), ("k", k, kshape), ("v", v, kshape), ("do", do, q.shape),
                          ("dq", dq, q.shape)),
                         ((B, H, bwd_rows_padded(N)), (("lse_log2", lse_log2), ("delta", delta))))
    scale = default_scale(d) if scale is None else float(scale)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
            lse_log2.data_ptr(), delta.data_ptr(), dq.data_ptr())
    tail = (scale, int(bool(causal)), _stream_handle(q.device, stream))
    if Nk == N:
        st = load().fa2_bwd_dq(*ptrs, B, H, N, d, *tail)
    else:
        st = load().fa2_bwd_dq_qk(*ptrs, B, H, N, Nk, d, *tail)
    _check(st, "fa2_bwd_dq")


def tile_config(d):
    vals = [_c_int() for _ in range(6)]
    _check(load().fa2_tile_config(d, *[ctypes.byref(x) for x in vals]), "fa2_tile_config")
    keys = ("fwd_block_q", "fwd_block_k", "bwd_block_k", "bwd_block_q", "fwd_waves", "bwd_waves")
    return dict(zip(keys, (x.value for x in vals)))
