"""Attention forward pass for AMD Instinct MI355X (gfx950).

Thin Python binding over ``libfa.so`` (C ABI declared in ``include/fa.h``):
argument marshalling only; every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.

    o, lse = tiled_attention_flash_amd.forward(q, k, v, causal=False, scale=None)

q ``[B, Lq, H, D]``, k/v ``[B, Lk, Hkv, D]``: contiguous fp16 tensors on the
current HIP device (BSHD layout), D in {64, 128}, H a multiple of Hkv.
Returns o ``[B, Lq, H, D]`` fp16 and lse ``[B, H, Lq]`` fp32 (natural-log
log-sum-exp of each row's scaled scores).  With Lq != Lk (or an explicit
``past_len``) query row i sits at key position i + past_len, default
Lk - Lq, which the causal mask uses.

    o, lse = tiled_attention_flash_amd.forward_splitkv(q, k, v, causal=False, scale=None)

computes the same result by splitting the keys over separate wavefronts and
merging the partial results (for few query rows against many keys); its fp32
workspace is allocated with torch unless one is passed.
``forward_splitkv_noalloc`` does the same with the library's static device
scratch instead of a workspace (for callers that cannot allocate).

    o, lse = tiled_attention_flash_amd.forward_fp8(q8, k8, v8, descale=(qd, kd, vd))

takes E4M3 inputs (one descale per tensor) and returns fp16 o, fp32 lse;

    dq, dk, dv, delta = tiled_attention_flash_amd.backward(q, k, v, o, lse, dout)

computes the gradients of sum(o * dout).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["forward", "forward_splitkv", "forward_splitkv_noalloc", "forward_fp8", "backward",
           "fa_fwd", "fa_fwd_kv", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "fa_fwd_fp8", "fa_bwd",
           "fa_bwd_kv",
           "fa_splitkv_splits", "fa_splitkv_workspace_bytes", "fa_status_string", "library",
           "library_path", "FaError", "STATUS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libfa.so")
_lib = None

STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULLPTR", 2: "FA_ERR_SHAPE", 3: "FA_ERR_GQA", 4: "FA_ERR_HEADDIM",
    5: "FA_ERR_SCALE", 6: "FA_ERR_ALIGN", 7: "FA_ERR_ALIAS", 8: "FA_ERR_LAUNCH",
    9: "FA_ERR_DEVICE", 10: "FA_ERR_WORKSPACE", 11: "FA_ERR_SCRATCH",
}

SPLITKV_SCRATCH_BYTES = 16 << 20  # FA_SPLITKV_SCRATCH_BYTES


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def library():
    """Load libfa.so.  There is no fallback: a missing library is an error."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m tiled_attention_flash_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    c_int = ctypes.c_int
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp] + [c_int] * 6 + [ctypes.c_float, vp]
    lib.fa_fwd.restype = c_int
    lib.fa_fwd_kv.argtypes = [vp, vp, vp, vp, vp] + [c_int] * 8 + [ctypes.c_float, vp]
    lib.fa_fwd_kv.restype = c_int
    lib.fa_fwd_splitkv.argtypes = ([vp, vp, vp, vp, vp] + [c_int] * 8 + [ctypes.c_float, c_int, vp,
                                                                          ctypes.c_longlong, vp])
    lib.fa_fwd_splitkv.restype = c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = ([vp, vp, vp, vp, vp] + [c_int] * 8 + [ctypes.c_float, c_int, vp])
    lib.fa_fwd_splitkv_noalloc.restype = c_int
    lib.fa_splitkv_splits.argtypes = [c_int] * 8
    lib.fa_splitkv_splits.restype = c_int
    lib.fa_splitkv_workspace_bytes.argtypes = [c_int] * 5
    lib.fa_splitkv_workspace_bytes.restype = ctypes.c_longlong
    lib.fa_fwd_fp8.argtypes = ([vp, vp, vp, vp, vp] + [c_int] * 8 + [ctypes.c_float] * 4 + [vp])
    lib.fa_fwd_fp8.restype = c_int
    lib.fa_bwd.argtypes = [vp] * 10 + [c_int] * 6 + [ctypes.c_float, vp]
    lib.fa_bwd.restype = c_int
    lib.fa_bwd_kv.argtypes = [vp] * 10 + [c_int] * 8 + [ctypes.c_float, vp]
    lib.fa_bwd_kv.restype = c_int
    lib.fa_status_string.argtypes = [c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = c_int
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return library().fa_status_string(int(status)).decode()


def fa_fwd(q, k, v, o, lse, B, L, H, Hkv, D, causal, scale, stream) -> int:
    """Direct call of the C entry point with raw addresses (ints or None).
    Returns the status code unchanged."""
    return int(library().fa_fwd(q, k, v, o, lse, int(B), int(L), int(H), int(Hkv), int(D),
                                int(bool(causal)), float(scale), stream))


def fa_fwd_kv(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale, stream) -> int:
    """Direct call of the C entry point for Lq != Lk; status returned unchanged."""
    return int(library().fa_fwd_kv(q, k, v, o, lse, int(B), int(Lq), int(Lk), int(H), int(Hkv),
                                   int(D), int(bool(causal)), int(past_len), float(scale), stream))


def fa_fwd_splitkv(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale, n_splits,
                   workspace, workspace_bytes, stream) -> int:
    """Direct call of the split-KV entry point; status returned unchanged."""
    return int(library().fa_fwd_splitkv(q, k, v, o, lse, int(B), int(Lq), int(Lk), int(H),
                                        int(Hkv), int(D), int(bool(causal)), int(past_len),
                                        float(scale), int(n_splits), workspace,
                                        int(workspace_bytes), stream))


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale,
                           n_splits, stream) -> int:
    """Direct call of the allocation-free split-KV entry point (static device
    scratch instead of a workspace); status returned unchanged."""
    return int(library().fa_fwd_splitkv_noalloc(q, k, v, o, lse, int(B), int(Lq), int(Lk), int(H),
                                                int(Hkv), int(D), int(bool(causal)), int(past_len),
                                                float(scale), int(n_splits), stream))


def fa_splitkv_splits(B, Lq, Lk, H, Hkv, D, causal, past_len) -> int:
    return int(library().fa_splitkv_splits(int(B), int(Lq), int(Lk), int(H), int(Hkv), int(D),
                                           int(bool(causal)), int(past_len)))


def fa_splitkv_workspace_bytes(B, Lq, H, D, n_splits) -> int:
    return int(library().fa_splitkv_workspace_bytes(int(B), int(Lq), int(H), int(D),
                                                    int(n_splits)))


def fa_fwd_fp8(q, k, v, o, lse, B, Lq, Lk, H, Hkv, D, causal, past_len, scale, q_descale,
               k_descale, v_descale, stream) -> int:
    return int(library().fa_fwd_fp8(q, k, v, o, lse, int(B), int(Lq), int(Lk), int(H), int(Hkv),
                                    int(D), int(bool(causal)), int(past_len), float(scale),
                                    float(q_descale), float(k_descale), float(v_descale), stream))


def forward_fp8(q, k, v, descale=(1.0, 1.0, 1.0), causal: bool = False,
                scale: float | None = None, out=None, lse=None, with_lse: bool = True,
                past_len: int | None = None):
    """Attention forward on E4M3 inputs (uint8 or float8_e4m3fn tensors, BSHD,
    contiguous) with per-tensor descales (q, k, v) on the current stream.
    Returns (o, lse): o float16 shaped like q, lse float32 [B, H, Lq] (None
    when ``with_lse`` is False and no buffer is given)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if (not isinstance(t, torch.Tensor) or t.dtype not in (torch.uint8, torch.float8_e4m3fn)
                or not t.is_cuda):
            raise TypeError(f"{name} must be a uint8 / float8_e4m3fn tensor on a HIP device")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D [B, L, heads, D] tensor")
    B, L, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")
    Lk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse = _outputs(q, out, lse, with_lse)
    past = Lk - L if past_len is None else int(past_len)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_fwd_fp8(q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None,
                        out.data_ptr() or None,
                        (lse.data_ptr() or None) if lse is not None else None, B, L, Lk, H, Hkv,
                        D, causal, past, scale, descale[0], descale[1], descale[2], stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out, lse


def _check_qkv(q, k, v):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_cuda:
            raise TypeError(f"{name} must be a float16 tensor on a HIP device")
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D [B, L, heads, D] tensor")
    B, L, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on the same device")


def _outputs(q, out, lse, with_lse):
    """Output buffers for a forward over q [B, L, H, D]: the caller's, checked
    against q's shape and device (o float16, lse float32 [B, H, L]), or new
    ones.  The kernels write B*L*H*D fp16 values and B*H*L fp32 values, so a
    smaller or misplaced buffer is rejected here, before any launch."""
    import torch

    B, L, H, D = q.shape
    if out is None:
        out = torch.empty((B, L, H, D), dtype=torch.float16, device=q.device)
    elif (not isinstance(out, torch.Tensor) or tuple(out.shape) != (B, L, H, D) or
          out.dtype != torch.float16 or not out.is_contiguous() or out.device != q.device):
        raise ValueError("out must be a contiguous float16 [B, L, H, D] tensor shaped like q on "
                         "q's device")
    if lse is None and with_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    elif lse is not None and (not isinstance(lse, torch.Tensor) or tuple(lse.shape) != (B, H, L) or
                              lse.dtype != torch.float32 or not lse.is_contiguous() or
                              lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, L] tensor on q's device")
    return out, lse


def forward_splitkv(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
                    with_lse: bool = True, past_len: int | None = None,
                    n_splits: int | None = None, workspace=None):
    """The forward pass by key splits plus a merge (fa_fwd_splitkv), on the
    current stream.  ``n_splits`` None lets the library choose; ``workspace``
    (a CUDA tensor of at least ``fa_splitkv_workspace_bytes`` bytes) is
    allocated here when not given.  Returns (o, lse) as ``forward`` does."""
    import torch

    _check_qkv(q, k, v)
    B, L, H, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse = _outputs(q, out, lse, with_lse)
    past = Lk - L if past_len is None else int(past_len)
    splits = fa_splitkv_splits(B, L, Lk, H, Hkv, D, causal, past) if n_splits is None else int(n_splits)
    need = fa_splitkv_workspace_bytes(B, L, H, D, max(splits, 1))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    ptrs = (q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None,
            out.data_ptr() or None, (lse.data_ptr() or None) if lse is not None else None)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_fwd_splitkv(*ptrs, B, L, Lk, H, Hkv, D, causal, past, scale, splits,
                            workspace.data_ptr() or None, ws_bytes, stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out, lse


def forward_splitkv_noalloc(q, k, v, causal: bool = False, scale: float | None = None, out=None,
                            lse=None, with_lse: bool = True, past_len: int | None = None,
                            n_splits: int | None = None):
    """forward_splitkv through fa_fwd_splitkv_noalloc: the library's static
    device scratch holds the partial results, so the call itself allocates
    nothing on the device (out and lse are allocated here only when not
    given).  Calls that overlap on one GPU race on that scratch."""
    import torch

    _check_qkv(q, k, v)
    B, L, H, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse = _outputs(q, out, lse, with_lse)
    past = Lk - L if past_len is None else int(past_len)
    splits = 0 if n_splits is None else int(n_splits)
    ptrs = (q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None,
            out.data_ptr() or None, (lse.data_ptr() or None) if lse is not None else None)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = fa_fwd_splitkv_noalloc(*ptrs, B, L, Lk, H, Hkv, D, causal, past, scale, splits, stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out, lse


def fa_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, B, L, H, Hkv, D, causal, scale,
           stream) -> int:
    """Direct call of the backward entry point; status returned unchanged."""
    return int(library().fa_bwd(q, k, v, o, dout, lse, delta, dq, dk, dv, int(B), int(L), int(H),
                                int(Hkv), int(D), int(bool(causal)), float(scale), stream))


def fa_bwd_kv(q, k, v, o, dout, lse, delta, dq, dk, dv, B, Lq, Lk, H, Hkv, D, causal, past_len,
              scale, stream) -> int:
    """Direct call of the backward entry point for Lq != Lk; status returned unchanged."""
    return int(library().fa_bwd_kv(q, k, v, o, dout, lse, delta, dq, dk, dv, int(B), int(Lq),
                                   int(Lk), int(H), int(Hkv), int(D), int(bool(causal)),
                                   int(past_len), float(scale), stream))


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, delta=None, past_len: int | None = None):
    """Gradients (dq, dk, dv) of sum(o * dout) for the forward that produced
    o and lse from q, k, v, on the current stream.  q, o, dout [B, Lq, H, D],
    k, v [B, Lk, Hkv, D]; with Lq != Lk (or an explicit ``past_len``) query
    row i sits at key position i + past_len, default Lk - Lq, as in
    ``forward``.  Output and Delta buffers are allocated with torch unless
    given; returns (dq, dk, dv, delta)."""
    import torch

    _check_qkv(q, k, v)
    B, L, H, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    past = Lk - L if past_len is None else int(past_len)
    for name, t in (("o", o), ("dout", dout)):
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or t.shape != q.shape or
                not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous float16 tensor shaped like q on q's device")
    for name, t in (("lse", lse), ("delta", delta)):
        if t is not None and (t.dtype != torch.float32 or t.shape != (B, H, L) or
                              not t.is_contiguous() or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous float32 [B, H, L] tensor on q's device")
    if lse is None:
        raise ValueError("lse is required")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    # the kernels write dq like q and dk, dv like k (fp16, BSHD, contiguous)
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t is not None and (not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or
                              t.shape != like.shape or not t.is_contiguous() or
                              t.device != q.device):
            raise ValueError(f"{name} must be a contiguous float16 tensor shaped like "
                             f"{'q' if like is q else 'k'} on q's device")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    delta = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if delta is None else delta
    ptrs = [t.data_ptr() or None for t in (q, k, v, o, dout, lse, delta, dq, dk, dv)]
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if Lk == L and past == 0:
            st = fa_bwd(*ptrs, B, L, H, Hkv, D, causal, scale, stream)
        else:
            st = fa_bwd_kv(*ptrs, B, L, Lk, H, Hkv, D, causal, past, scale, stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return dq, dk, dv, delta


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
            with_lse: bool = True, past_len: int | None = None):
    """Attention forward on the current stream.  Returns (o, lse); lse is None
    when ``with_lse`` is False and no ``lse`` buffer is given."""
    import torch

    _check_qkv(q, k, v)
    B, L, H, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out, lse = _outputs(q, out, lse, with_lse)
    past = Lk - L if past_len is None else int(past_len)
    ptrs = (q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None,
            out.data_ptr() or None, (lse.data_ptr() or None) if lse is not None else None)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if Lk == L and past == 0:
            st = fa_fwd(*ptrs, B, L, H, Hkv, D, causal, scale, stream)
        else:
            st = fa_fwd_kv(*ptrs, B, L, Lk, H, Hkv, D, causal, past, scale, stream)
    if st != 0:
        raise FaError(st, fa_status_string(st))
    return out, lse
