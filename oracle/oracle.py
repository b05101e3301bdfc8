"""ctypes wrapper around ``libfa_oracle.so`` (built from ``fa_oracle.c`` by gcc).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Every function takes fp16 inputs as numpy ``float16`` arrays or torch CPU
``float16`` tensors in BSHD layout (q ``[B, L, H, D]``, k/v ``[B, L, Hkv, D]``)
and returns float64 numpy arrays: o ``[B, L, H, D]`` and lse ``[B, H, L]``.
The arithmetic is the plain three-step attention definition in fp64; the
citations are in ``fa_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB = os.path.join(_HERE, "libfa_oracle.so")
_lib = None


def library_path() -> str:
    return _LIB


def build() -> str:
    """Compile the oracle with gcc (-O3, no -ffast-math: fixed summation order)."""
    cmd = ["gcc", "-O3", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", "-pthread",
           _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    c_int, c_long, c_double = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.fa_oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.fa_oracle_half_to_double.restype = c_double
    lib.fa_oracle_fwd.argtypes = [u16p, u16p, u16p, f64p, f64p] + [c_int] * 6 + [c_double, c_int]
    lib.fa_oracle_fwd.restype = c_int
    lib.fa_oracle_rows.argtypes = ([u16p, u16p, u16p] + [c_int] * 6 +
                                  [c_double, i64p, c_long, f64p, f64p, c_int])
    lib.fa_oracle_rows.restype = c_int
    lib.fa_oracle_row_probs.argtypes = ([u16p, u16p, u16p] + [c_int] * 6 +
                                       [c_double, c_int, c_int, c_int, f64p])
    lib.fa_oracle_row_probs.restype = c_int
    lib.fa_oracle_fwd_kv.argtypes = ([u16p, u16p, u16p, f64p, f64p] + [c_int] * 8 +
                                     [c_double, c_int])
    lib.fa_oracle_fwd_kv.restype = c_int
    lib.fa_oracle_rows_kv.argtypes = ([u16p, u16p, u16p] + [c_int] * 8 +
                                      [c_double, i64p, c_long, f64p, f64p, c_int])
    lib.fa_oracle_rows_kv.restype = c_int
    lib.fa_oracle_row_probs_kv.argtypes = ([u16p, u16p, u16p] + [c_int] * 8 +
                                           [c_double, c_int, c_int, c_int, f64p])
    lib.fa_oracle_row_probs_kv.restype = c_int
    lib.fa_oracle_bwd.argtypes = ([u16p, u16p, u16p, u16p, f64p, f64p, f64p] + [c_int] * 6 +
                                  [c_double, c_int])
    lib.fa_oracle_bwd.restype = c_int
    lib.fa_oracle_bwd_kv.argtypes = ([u16p, u16p, u16p, u16p, f64p, f64p, f64p] + [c_int] * 8 +
                                     [c_double, c_int])
    lib.fa_oracle_bwd_kv.restype = c_int
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.fa_oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.fa_oracle_e4m3_to_double.restype = c_double
    lib.fa_oracle_fwd_fp8.argtypes = ([u8p, u8p, u8p, f64p, f64p, f64p] + [c_int] * 8 +
                                      [c_double] * 7 + [c_int])
    lib.fa_oracle_fwd_fp8.restype = c_int
    lib.fa_oracle_rows_fp8.argtypes = ([u8p, u8p, u8p] + [c_int] * 8 + [c_double] * 7 +
                                       [i64p, c_long, f64p, f64p, f64p, c_int])
    lib.fa_oracle_rows_fp8.restype = c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = _bind(_LIB)
    return _lib


def _as_half_bits(x) -> np.ndarray:
    """fp16 array/tensor -> contiguous uint16 numpy view of its bit patterns."""
    if hasattr(x, "detach"):  # torch tensor; only the bits are taken, no torch math
        x = x.detach()
        if x.device.type != "cpu":
            raise ValueError("oracle inputs must live in host memory")
        x = x.contiguous().view(dtype=__import__("torch").int16).numpy()
    a = np.ascontiguousarray(x)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    elif a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"oracle inputs must be float16, got {a.dtype}")
    return a


def _shape(q, k, v):
    """q [B, Lq, H, D], k and v [B, Lk, Hkv, D] (Lq and Lk may differ)."""
    q, k, v = _as_half_bits(q), _as_half_bits(k), _as_half_bits(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D BSHD")
    B, Lq, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Lk, Hkv = k.shape[1], k.shape[2]
    if Hkv <= 0 or H % Hkv:
        raise ValueError(f"H={H} is not a multiple of Hkv={Hkv}")
    return q, k, v, B, Lq, Lk, H, Hkv, D


def default_past_len(Lq: int, Lk: int) -> int:
    """Position of query row 0 in the key sequence when none is given: the
    queries are the last Lq positions of the Lk keys (a prefill after a
    cached prefix), so past_len = Lk - Lq; 0 when the lengths are equal."""
    return Lk - Lq


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_scale(D: int) -> float:
    """1/sqrt(dim): the scale the TileLang AMD page's kernel sets up in its
    section on initialisation and kernel entry."""
    return 1.0 / float(np.sqrt(D))


def forward(q, k, v, causal: bool = False, scale: float | None = None, nthreads: int = 0,
            lib=None, past_len: int | None = None):
    """Full attention forward in fp64. Returns (o [B,Lq,H,D], lse [B,H,Lq]).
    Under the causal mask query row i sits at position i + past_len of the
    keys (default Lk - Lq).  ``lib`` selects another build of the same source
    (used by the tests that check the pins reject deliberately broken copies
    of the oracle)."""
    lib = lib or _load()
    q, k, v, B, Lq, Lk, H, Hkv, D = _shape(q, k, v)
    scale = default_scale(D) if scale is None else float(scale)
    past = default_past_len(Lq, Lk) if past_len is None else int(past_len)
    o = np.empty((B, Lq, H, D), np.float64)
    lse = np.empty((B, H, Lq), np.float64)
    if Lq == Lk and past == 0:
        rc = lib.fa_oracle_fwd(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                               _ptr(v, ctypes.c_uint16), _ptr(o, ctypes.c_double),
                               _ptr(lse, ctypes.c_double), B, Lq, H, Hkv, D, int(bool(causal)),
                               scale, int(nthreads))
    else:
        rc = lib.fa_oracle_fwd_kv(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                  _ptr(v, ctypes.c_uint16), _ptr(o, ctypes.c_double),
                                  _ptr(lse, ctypes.c_double), B, Lq, Lk, H, Hkv, D,
                                  int(bool(causal)), past, scale, int(nthreads))
    if rc:
        raise ValueError("oracle rejected the problem")
    return o, lse


def rows(q, k, v, row_ids, causal: bool = False, scale: float | None = None, nthreads: int = 0,
         lib=None, past_len: int | None = None):
    """Selected rows: row_ids is an int array of (b, h, i) triples, shape [n, 3].
    Returns (o_rows [n, D], lse_rows [n])."""
    lib = lib or _load()
    q, k, v, B, Lq, Lk, H, Hkv, D = _shape(q, k, v)
    scale = default_scale(D) if scale is None else float(scale)
    past = default_past_len(Lq, Lk) if past_len is None else int(past_len)
    r = np.ascontiguousarray(np.asarray(row_ids, dtype=np.int64).reshape(-1, 3))
    n = r.shape[0]
    o = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib.fa_oracle_rows_kv(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                               _ptr(v, ctypes.c_uint16), B, Lq, Lk, H, Hkv, D, int(bool(causal)),
                               past, scale, _ptr(r, ctypes.c_int64), n, _ptr(o, ctypes.c_double),
                               _ptr(lse, ctypes.c_double), int(nthreads))
    if rc:
        raise ValueError("oracle rejected the rows")
    return o, lse


def row_probs(q, k, v, b: int, h: int, i: int, causal: bool = False, scale: float | None = None,
              lib=None, past_len: int | None = None):
    """Softmax probabilities of row (b, h, i) over all Lk keys (0 where masked)."""
    lib = lib or _load()
    q, k, v, B, Lq, Lk, H, Hkv, D = _shape(q, k, v)
    scale = default_scale(D) if scale is None else float(scale)
    past = default_past_len(Lq, Lk) if past_len is None else int(past_len)
    p = np.empty((Lk,), np.float64)
    rc = lib.fa_oracle_row_probs_kv(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                    _ptr(v, ctypes.c_uint16), B, Lq, Lk, H, Hkv, D,
                                    int(bool(causal)), past, scale, b, h, i,
                                    _ptr(p, ctypes.c_double))
    if rc:
        raise ValueError("oracle rejected the row")
    return p


def backward(q, k, v, dout, causal: bool = False, scale: float | None = None, nthreads: int = 0,
             lib=None, past_len: int | None = None):
    """Gradients of sum(O * dout) in fp64.  q, dout [B, Lq, H, D], k, v
    [B, Lk, Hkv, D] (float16); under the causal mask query row i sits at
    position i + past_len (default Lk - Lq) and keeps key j iff
    i + past_len >= j, as in `forward`.  Returns (dq [B,Lq,H,D],
    dk [B,Lk,Hkv,D], dv [B,Lk,Hkv,D]) as float64 arrays."""
    lib = lib or _load()
    q, k, v, B, Lq, Lk, H, Hkv, D = _shape(q, k, v)
    do = _as_half_bits(dout)
    if do.shape != q.shape:
        raise ValueError(f"dout {do.shape} must be shaped like q {q.shape}")
    scale = default_scale(D) if scale is None else float(scale)
    past = default_past_len(Lq, Lk) if past_len is None else int(past_len)
    dq = np.empty((B, Lq, H, D), np.float64)
    dk = np.empty((B, Lk, Hkv, D), np.float64)
    dv = np.empty((B, Lk, Hkv, D), np.float64)
    rc = lib.fa_oracle_bwd_kv(_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                              _ptr(v, ctypes.c_uint16), _ptr(do, ctypes.c_uint16),
                              _ptr(dq, ctypes.c_double), _ptr(dk, ctypes.c_double),
                              _ptr(dv, ctypes.c_double), B, Lq, Lk, H, Hkv, D, int(bool(causal)),
                              past, scale, int(nthreads))
    if rc:
        raise ValueError("oracle rejected the problem")
    return dq, dk, dv


def _as_fp8_codes(x) -> np.ndarray:
    """E4M3 codes (torch float8_e4m3fn/uint8 tensor or uint8 array) ->
    contiguous uint8 numpy array; only the bytes are taken."""
    if hasattr(x, "detach"):
        x = x.detach()
        if x.device.type != "cpu":
            raise ValueError("oracle inputs must live in host memory")
        x = x.contiguous().view(dtype=__import__("torch").uint8).numpy()
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint8:
        raise TypeError(f"fp8 oracle inputs must be E4M3 bytes, got {a.dtype}")
    return a


def _shape8(q, k, v):
    q, k, v = _as_fp8_codes(q), _as_fp8_codes(k), _as_fp8_codes(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D BSHD")
    B, Lq, H, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    Lk, Hkv = k.shape[1], k.shape[2]
    if Hkv <= 0 or H % Hkv:
        raise ValueError(f"H={H} is not a multiple of Hkv={Hkv}")
    return q, k, v, B, Lq, Lk, H, Hkv, D


def forward_fp8(q, k, v, descale=(1.0, 1.0, 1.0), causal: bool = False,
                scale: float | None = None, past_len: int | None = None, bound_model=None,
                nthreads: int = 0, lib=None):
    """fp8 forward in fp64 on the decoded values descale * e4m3(code).
    q [B,Lq,H,D], k/v [B,Lk,Hkv,D] E4M3 codes; descale = (q, k, v) factors.
    Returns (o [B,Lq,H,D], lse [B,H,Lq], bound [B,Lq,H,D] or None): bound is
    the largest change of O that rounding the probabilities under
    ``bound_model`` = (rel, floor, abs) can cause (see fa_oracle.c)."""
    lib = lib or _load()
    q, k, v, B, Lq, Lk, H, Hkv, D = _shape8(q, k, v)
    scale = default_scale(D) if scale is None else float(scale)
    past = default_past_len(Lq, Lk) if past_len is None else int(past_len)
    o = np.empty((B, Lq, H, D), np.float64)
    lse = np.empty((B, H, Lq), np.float64)
    bound = np.empty((B, Lq, H, D), np.float64) if bound_model is not None else None
    rel, floor, ab = bound_model if bound_model is not None else (0.0, 0.0, 0.0)
    u8 = ctypes.c_uint8
    rc = lib.fa_oracle_fwd_fp8(_ptr(q, u8), _ptr(k, u8), _ptr(v, u8), _ptr(o, ctypes.c_double),
                               _ptr(lse, ctypes.c_double),
                               _ptr(bound, ctypes.c_double) if bound is not None else None,
                               B, Lq, Lk, H, Hkv, D, int(bool(causal)), past, scale,
                               float(descale[0]), float(descale[1]), float(descale[2]),
                               float(rel), float(floor), float(ab), int(nthreads))
    if rc:
        raise ValueError("oracle rejected the problem")
    return o, lse, bound


def rows_fp8(q, k, v, row_ids, descale=(1.0, 1.0, 1.0), causal: bool = False,
             scale: float | None = None, past_len: int | None = None, bound_model=None,
             nthreads: int = 0, lib=None):
    """Selected rows of forward_fp8: row_ids [n, 3] of (b, h, i).
    Returns (o_rows [n, D], lse_rows [n], bound_rows [n, D] or None)."""
    lib = lib or _load()
    q, k, v, B, Lq, Lk, H, Hkv, D = _shape8(q, k, v)
    scale = default_scale(D) if scale is None else float(scale)
    past = default_past_len(Lq, Lk) if past_len is None else int(past_len)
    r = np.ascontiguousarray(np.asarray(row_ids, dtype=np.int64).reshape(-1, 3))
    n = r.shape[0]
    o = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    bound = np.empty((n, D), np.float64) if bound_model is not None else None
    rel, floor, ab = bound_model if bound_model is not None else (0.0, 0.0, 0.0)
    u8 = ctypes.c_uint8
    rc = lib.fa_oracle_rows_fp8(_ptr(q, u8), _ptr(k, u8), _ptr(v, u8), B, Lq, Lk, H, Hkv, D,
                                int(bool(causal)), past, scale, float(descale[0]),
                                float(descale[1]), float(descale[2]), float(rel), float(floor),
                                float(ab), _ptr(r, ctypes.c_int64), n, _ptr(o, ctypes.c_double),
                                _ptr(lse, ctypes.c_double),
                                _ptr(bound, ctypes.c_double) if bound is not None else None,
                                int(nthreads))
    if rc:
        raise ValueError("oracle rejected the rows")
    return o, lse, bound


def e4m3_to_double(code: int, lib=None) -> float:
    """The oracle's own E4M3 decoder, exposed so it can be pinned."""
    lib = lib or _load()
    return float(lib.fa_oracle_e4m3_to_double(int(code) & 0xFF))


def half_to_double(bits: int, lib=None) -> float:
    """The oracle's own binary16 decoder, exposed so it can be pinned."""
    lib = lib or _load()
    return float(lib.fa_oracle_half_to_double(int(bits) & 0xFFFF))


def build_variant(src_text: str, out_path: str):
    """Compile `src_text` (a modified copy of fa_oracle.c) to `out_path` and
    bind it.  Only the tests use this, to show that each pin rejects a
    plausible mistake planted in a copy of the oracle."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-pthread", src, "-o",
                    out_path, "-lm"], check=True)
    return _bind(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()
