"""CPU oracle for the sequence-parallel region -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The HIP library never calls it and shares no code with it.

`fwd` / `bwd` wrap the plain C definition in sp_oracle.c (see its header for the
pages' passages and the readings taken).  Arrays are numpy: bf16 activations
are passed as uint16 bit patterns, fp32 as float32, the exact mode as float64.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F64 = 0, 1, 2
RMSNORM, LAYERNORM = 0, 1

_NP_DTYPE = {F32: np.float32, BF16: np.uint16, F64: np.float64}


class Desc(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int64), ("B", ctypes.c_int64), ("H", ctypes.c_int64),
        ("T", ctypes.c_int32), ("j", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("norm", ctypes.c_int32),
        ("eps", ctypes.c_float), ("p", ctypes.c_float),
        ("seed", ctypes.c_uint64),
    ]


_lib = None


def lib():
    """Load oracle/libsp_oracle.so, building it with gcc if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        vp, i64, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64
        L.sp_oracle_fwd.argtypes = [ctypes.POINTER(Desc), i64, i64, ctypes.POINTER(vp), vp,
                                    vp, vp, vp, vp, vp, vp, vp]
        L.sp_oracle_fwd.restype = ctypes.c_int
        L.sp_oracle_bwd.argtypes = [ctypes.POINTER(Desc), i64, i64, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, vp, vp]
        L.sp_oracle_bwd.restype = ctypes.c_int
        L.sp_oracle_uniform_words.argtypes = [u64, u64, i64, vp]
        L.sp_oracle_uniform_words.restype = None
        L.sp_oracle_keep_mask.argtypes = [u64, ctypes.c_float, u64, i64, vp]
        L.sp_oracle_keep_mask.restype = None
        L.sp_oracle_f32_to_bf16.argtypes = [vp, i64, vp]
        L.sp_oracle_f32_to_bf16.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def make_desc(S, B, H, T, j, dtype, norm, eps, p, seed):
    return Desc(S, B, H, T, j, dtype, norm, eps, p, seed)


def fwd(desc, P_rows, residual, gamma, beta=None, row0=0, nrows=None):
    """Forward of the SP region over shard rows [row0, row0+nrows).

    P_rows: list of T arrays, each (nrows, H) = rows row0.. of P_t^(j).
    residual: (nrows, H).  gamma/beta: (H,) (converted to float64 exactly).
    Returns dict h, y, mask, mean (LayerNorm) / None, rstd (float64).
    """
    R = (desc.S // desc.T) * desc.B
    if nrows is None:
        nrows = R - row0
    H = desc.H
    et = _NP_DTYPE[desc.dtype]
    P_rows = [_c(np.reshape(x, (nrows, H)), et) for x in P_rows]
    assert len(P_rows) == desc.T
    residual = _c(np.reshape(residual, (nrows, H)), et)
    gamma = _c(gamma, np.float64)
    beta = _c(beta, np.float64)
    h = np.empty((nrows, H), et)
    y = np.empty((nrows, H), et)
    mask = np.empty((nrows, H), np.uint8)
    mean = np.empty(nrows, np.float64) if desc.norm == LAYERNORM else None
    rstd = np.empty(nrows, np.float64)
    parr = (ctypes.c_void_p * desc.T)(*[x.ctypes.data for x in P_rows])
    rc = lib().sp_oracle_fwd(ctypes.byref(desc), row0, nrows, parr, _ptr(residual), _ptr(gamma),
                             _ptr(beta), _ptr(h), _ptr(y), _ptr(mask), _ptr(mean), _ptr(rstd))
    if rc != 0:
        raise ValueError(f"sp_oracle_fwd rejected its arguments ({rc})")
    return {"h": h, "y": y, "mask": mask, "mean": mean, "rstd": rstd}


def bwd(desc, dY, h, mask, mean, rstd, gamma, dR=None, row0=0, nrows=None):
    """Backward of the SP region over shard rows [row0, row0+nrows).

    Returns dict d_res, dP (activation type), dgamma, dbeta (float64 sums over
    these rows; dbeta None for RMSNorm).
    """
    R = (desc.S // desc.T) * desc.B
    if nrows is None:
        nrows = R - row0
    H = desc.H
    et = _NP_DTYPE[desc.dtype]
    dY = _c(np.reshape(dY, (nrows, H)), et)
    h = _c(np.reshape(h, (nrows, H)), et)
    dR = None if dR is None else _c(np.reshape(dR, (nrows, H)), et)
    mask = _c(np.reshape(mask, (nrows, H)), np.uint8)
    mean = _c(mean, np.float64)
    rstd = _c(rstd, np.float64)
    gamma = _c(gamma, np.float64)
    d_res = np.empty((nrows, H), et)
    dP = np.empty((nrows, H), et)
    dgamma = np.empty(H, np.float64)
    dbeta = np.empty(H, np.float64) if desc.norm == LAYERNORM else None
    rc = lib().sp_oracle_bwd(ctypes.byref(desc), row0, nrows, _ptr(dY), _ptr(h), _ptr(mask),
                             _ptr(mean), _ptr(rstd), _ptr(gamma), _ptr(dR), _ptr(d_res),
                             _ptr(dP), _ptr(dgamma), _ptr(dbeta))
    if rc != 0:
        raise ValueError(f"sp_oracle_bwd rejected its arguments ({rc})")
    return {"d_res": d_res, "dP": dP, "dgamma": dgamma, "dbeta": dbeta}


def uniform_words(seed, start, n):
    out = np.empty(n, np.uint32)
    lib().sp_oracle_uniform_words(seed, start, n, _ptr(out))
    return out


def keep_mask(seed, p, start, n):
    out = np.empty(n, np.uint8)
    lib().sp_oracle_keep_mask(seed, p, start, n, _ptr(out))
    return out


def f32_to_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().sp_oracle_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(b):
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)
