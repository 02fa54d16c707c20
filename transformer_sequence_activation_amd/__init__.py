"""Python binding of libsp_region.so, the MI355X sequence-parallel region kernels.

Argument marshalling only: every step of the forward and backward runs in the
HIP kernels of csrc/sp_region.hip.  PyTorch supplies device memory and the
stream.  The C entry points are exposed under their C names
(`sp_region_fwd`, `sp_region_bwd`, `sp_region_bwd_noalloc`,
`sp_region_bwd_workspace_size`, `sp_region_bwd_schedule`, `sp_region_traffic_bytes`,
`sp_region_strerror`, `sp_region_version`); `forward`
and `backward` allocate the outputs with torch and call them.

If the shared library is missing, `load()` raises: there is no fallback path.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsp_region.so")

SP_MAX_T = 64
SP_F32, SP_BF16 = 0, 1
SP_RMSNORM, SP_LAYERNORM = 0, 1
SP_FLAG_RECOMPUTE_MASK = 1
SP_OK = 0
SP_NOALLOC_SCRATCH_BYTES = 32 << 20
STATUS = {0: "SP_OK", -1: "SP_EINVAL", -2: "SP_ESHAPE", -3: "SP_EDTYPE", -4: "SP_EPARAM",
          -5: "SP_EALIGN", -6: "SP_EWORKSPACE", -7: "SP_EHIP", -8: "SP_ESCRATCH"}
EXPORTED = ("sp_region_fwd", "sp_region_bwd", "sp_region_bwd_noalloc", "sp_region_bwd_workspace_size",
            "sp_region_bwd_schedule", "sp_region_traffic_bytes", "sp_region_strerror",
            "sp_region_version")


class SpDesc(ctypes.Structure):
    """sp_desc_t of include/sp_region.h."""
    _fields_ = [
        ("S", ctypes.c_int64), ("B", ctypes.c_int64), ("H", ctypes.c_int64),
        ("T", ctypes.c_int32), ("j", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("norm", ctypes.c_int32),
        ("eps", ctypes.c_float), ("p", ctypes.c_float),
        ("seed", ctypes.c_uint64),
        ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
    ]

    @property
    def R(self):
        return (self.S // self.T) * self.B if self.T > 0 else 0


class SpRegionError(RuntimeError):
    def __init__(self, status, text):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


_lib = None


def load(path=LIB_PATH):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m transformer_sequence_activation_amd.build`")
    L = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    pdesc = ctypes.POINTER(SpDesc)
    L.sp_region_fwd.argtypes = [pdesc, ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.sp_region_fwd.restype = ctypes.c_int
    L.sp_region_bwd.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sp_region_bwd.restype = ctypes.c_int
    L.sp_region_bwd_noalloc.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.sp_region_bwd_noalloc.restype = ctypes.c_int
    L.sp_region_bwd_workspace_size.argtypes = [pdesc]
    L.sp_region_bwd_workspace_size.restype = sz
    L.sp_region_bwd_schedule.argtypes = [pdesc]
    L.sp_region_bwd_schedule.restype = ctypes.c_int
    L.sp_region_traffic_bytes.argtypes = [pdesc, ctypes.POINTER(ctypes.c_uint64),
                                          ctypes.POINTER(ctypes.c_uint64)]
    L.sp_region_traffic_bytes.restype = ctypes.c_int
    L.sp_region_strerror.argtypes = [ctypes.c_int]
    L.sp_region_strerror.restype = ctypes.c_char_p
    L.sp_region_version.argtypes = []
    L.sp_region_version.restype = ctypes.c_int
    _lib = L
    return L


def make_desc(S, B, H, T, j, dtype="bf16", norm="rms", eps=1e-6, p=0.1, seed=1234, flags=0):
    dt = {"bf16": SP_BF16, "f32": SP_F32}.get(dtype, dtype)
    nm = {"rms": SP_RMSNORM, "ln": SP_LAYERNORM}.get(norm, norm)
    return SpDesc(S, B, H, T, j, dt, nm, eps, p, seed, flags, 0)


def _ptr(x):
    """Device address of a tensor (or an int address / None).  A tensor must be
    in GPU memory: the library would otherwise read a host address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("tensor arguments must be in GPU memory")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != SP_OK:
        raise SpRegionError(status, sp_region_strerror(status))


# ---- the C entry points, same names, tensors or raw addresses in ----

def sp_region_version():
    return load().sp_region_version()


def sp_region_strerror(status):
    return load().sp_region_strerror(status).decode()


def sp_region_traffic_bytes(desc):
    f, b = ctypes.c_uint64(), ctypes.c_uint64()
    _check(load().sp_region_traffic_bytes(ctypes.byref(desc), ctypes.byref(f), ctypes.byref(b)))
    return f.value, b.value


def sp_region_bwd_workspace_size(desc):
    return load().sp_region_bwd_workspace_size(ctypes.byref(desc))


def sp_region_bwd_schedule(desc):
    """0 = partial rows + finish kernel; k >= 1 = column workgroups with k row
    segments per strip; negative = status of a bad descriptor."""
    return load().sp_region_bwd_schedule(ctypes.byref(desc))


def sp_region_fwd(desc, P, residual, gamma, beta, h_out, y_out, mask_out, mean_out, rstd_out,
                  stream=None):
    """Returns the status code (0 = success); see include/sp_region.h."""
    parr = (ctypes.c_void_p * max(1, len(P)))(*[_ptr(x) for x in P])
    return load().sp_region_fwd(ctypes.byref(desc), parr, _ptr(residual), _ptr(gamma), _ptr(beta),
                                _ptr(h_out), _ptr(y_out), _ptr(mask_out), _ptr(mean_out),
                                _ptr(rstd_out), _stream(stream))


def sp_region_bwd(desc, dY, h, mask, mean, rstd, gamma, dR, d_residual, dP, dgamma, dbeta,
                  workspace, workspace_bytes, stream=None):
    """Returns the status code (0 = success); see include/sp_region.h."""
    return load().sp_region_bwd(ctypes.byref(desc), _ptr(dY), _ptr(h), _ptr(mask), _ptr(mean),
                                _ptr(rstd), _ptr(gamma), _ptr(dR), _ptr(d_residual), _ptr(dP),
                                _ptr(dgamma), _ptr(dbeta), _ptr(workspace), workspace_bytes,
                                _stream(stream))


def sp_region_bwd_noalloc(desc, dY, h, mask, mean, rstd, gamma, dR, d_residual, dP, dgamma, dbeta,
                          stream=None):
    """Returns the status code (0 = success); see include/sp_region.h."""
    return load().sp_region_bwd_noalloc(ctypes.byref(desc), _ptr(dY), _ptr(h), _ptr(mask), _ptr(mean),
                                        _ptr(rstd), _ptr(gamma), _ptr(dR), _ptr(d_residual), _ptr(dP),
                                        _ptr(dgamma), _ptr(dbeta), _stream(stream))


# ---- convenience wrappers: allocate outputs with torch, raise on error ----

def _act_dtype(desc):
    import torch
    return torch.bfloat16 if desc.dtype == SP_BF16 else torch.float32


def _need(name, t, dtype, numel, device):
    """Reject what the library cannot check itself: a missing tensor, the wrong
    dtype, device or size, or a non-contiguous layout."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def _on_stream(stream):
    """The torch stream to allocate and launch on (torch's current one by default)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def forward(desc, P, residual, gamma, beta=None, stream=None):
    """P: T full [S,B,H] device tensors; residual: the shard (R*H elements).
    Returns dict h, y, mask (None with SP_FLAG_RECOMPUTE_MASK), mean (None for
    RMSNorm), rstd.  Outputs are allocated, and the kernel enqueued, on `stream`
    (torch's current stream by default)."""
    import torch
    R, H = desc.R, desc.H
    act = _act_dtype(desc)
    if len(P) != desc.T:
        raise ValueError(f"P holds {len(P)} partials, the descriptor says T = {desc.T}")
    dev = residual.device
    if dev.type != "cuda":
        raise ValueError("tensors must be in GPU memory")
    for t, x in enumerate(P):
        _need(f"P[{t}]", x, act, desc.S * desc.B * H, dev)
    _need("residual", residual, act, R * H, dev)
    _need("gamma", gamma, torch.float32, H, dev)
    if desc.norm == SP_LAYERNORM:
        _need("beta", beta, torch.float32, H, dev)
    elif beta is not None:
        raise ValueError("beta must be None for RMSNorm")
    keep_mask = not (desc.flags & SP_FLAG_RECOMPUTE_MASK)
    s = _on_stream(stream)
    with torch.cuda.stream(s):
        out = {
            "h": torch.empty((R, H), dtype=act, device=dev),
            "y": torch.empty((R, H), dtype=act, device=dev),
            "mask": torch.empty((R, H), dtype=torch.uint8, device=dev) if keep_mask else None,
            "mean": torch.empty(R, dtype=torch.float32, device=dev) if desc.norm == SP_LAYERNORM else None,
            "rstd": torch.empty(R, dtype=torch.float32, device=dev),
        }
        _check(sp_region_fwd(desc, P, residual, gamma, beta, out["h"], out["y"], out["mask"],
                             out["mean"], out["rstd"], s))
    return out


def backward(desc, dY, h, mask, mean, rstd, gamma, dR=None, workspace=None, stream=None):
    """Returns dict d_res, dP, dgamma, dbeta (None for RMSNorm).  A workspace
    passed in must have been zero-filled before its first use; without one, a
    zero-filled workspace is allocated on `stream`, where the outputs are
    allocated and the kernels enqueued (torch's current stream by default)."""
    import torch
    R, H = desc.R, desc.H
    act = _act_dtype(desc)
    dev = dY.device
    if dev.type != "cuda":
        raise ValueError("tensors must be in GPU memory")
    _need("dY", dY, act, R * H, dev)
    _need("h", h, act, R * H, dev)
    if desc.flags & SP_FLAG_RECOMPUTE_MASK:
        if mask is not None:
            raise ValueError("mask must be None with SP_FLAG_RECOMPUTE_MASK")
    else:
        _need("mask", mask, torch.uint8, R * H, dev)
    if desc.norm == SP_LAYERNORM:
        _need("mean", mean, torch.float32, R, dev)
    elif mean is not None:
        raise ValueError("mean must be None for RMSNorm")
    _need("rstd", rstd, torch.float32, R, dev)
    _need("gamma", gamma, torch.float32, H, dev)
    if dR is not None:
        _need("dR", dR, act, R * H, dev)
    ws_bytes = sp_region_bwd_workspace_size(desc)
    if workspace is not None:
        if workspace.device != dev or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
        if workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError(f"workspace must hold at least {ws_bytes} bytes")
    s = _on_stream(stream)
    with torch.cuda.stream(s):
        if workspace is None:
            workspace = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        out = {
            "d_res": torch.empty((R, H), dtype=act, device=dev),
            "dP": torch.empty((R, H), dtype=act, device=dev),
            "dgamma": torch.empty(H, dtype=torch.float32, device=dev),
            "dbeta": torch.empty(H, dtype=torch.float32, device=dev) if desc.norm == SP_LAYERNORM else None,
        }
        _check(sp_region_bwd(desc, dY, h, mask, mean, rstd, gamma, dR, out["d_res"], out["dP"],
                             out["dgamma"], out["dbeta"], workspace,
                             workspace.numel() * workspace.element_size(), s))
    return out


class PreparedCall:
    """A C entry point with its arguments marshalled once, for tight timing loops.
    Calling it returns nothing and raises on a nonzero status."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep  # keeps ctypes objects and tensors alive

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != SP_OK:
            _check(rc)


def prepare_fwd(desc, P, residual, gamma, beta, h_out, y_out, mask_out, mean_out, rstd_out,
                stream=None):
    L = load()
    d = SpDesc.from_buffer_copy(desc)
    parr = (ctypes.c_void_p * len(P))(*[_ptr(x) for x in P])
    vp = ctypes.c_void_p
    args = (ctypes.byref(d), parr, vp(_ptr(residual)), vp(_ptr(gamma)), vp(_ptr(beta)),
            vp(_ptr(h_out)), vp(_ptr(y_out)), vp(_ptr(mask_out)), vp(_ptr(mean_out)),
            vp(_ptr(rstd_out)), vp(_stream(stream)))
    return PreparedCall(L.sp_region_fwd, args, (d, parr, P, residual, gamma, beta, h_out, y_out,
                                                mask_out, mean_out, rstd_out))


def prepare_bwd(desc, dY, h, mask, mean, rstd, gamma, dR, d_residual, dP, dgamma, dbeta,
                workspace, workspace_bytes, stream=None):
    L = load()
    d = SpDesc.from_buffer_copy(desc)
    vp = ctypes.c_void_p
    args = (ctypes.byref(d), vp(_ptr(dY)), vp(_ptr(h)), vp(_ptr(mask)), vp(_ptr(mean)),
            vp(_ptr(rstd)), vp(_ptr(gamma)), vp(_ptr(dR)), vp(_ptr(d_residual)), vp(_ptr(dP)),
            vp(_ptr(dgamma)), vp(_ptr(dbeta)), vp(_ptr(workspace)), ctypes.c_size_t(workspace_bytes),
            vp(_stream(stream)))
    return PreparedCall(L.sp_region_bwd, args, (d, dY, h, mask, mean, rstd, gamma, dR, d_residual,
                                                dP, dgamma, dbeta, workspace))
