"""ctypes binding of libm3.so: torch tensors in, the C entry points of include/m3.h called.

Argument marshalling only: shapes and dtypes are read off the tensors, outputs
and the workspace are allocated with torch (device memory is torch's job), and
the call goes to the HIP library on torch's current stream. There is no other
implementation behind these functions: if libm3.so is missing they raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; M3_LIBRARY names another build of the same ABI (the
# host-only sanitizer build of the tests)
LIB_PATH = os.environ.get("M3_LIBRARY") or os.path.join(HERE, "libm3.so")

M3_F32, M3_BF16 = 0, 1
M3_PATH_GENERIC, M3_PATH_MFMA, M3_PATH_SCAN = 0, 1, 2
STATUS = {0: "M3_OK", 1: "M3_EINVAL", 2: "M3_ESHAPE", 3: "M3_EDTYPE", 4: "M3_EALIGN",
          5: "M3_EUNSUPPORTED", 6: "M3_EHIP", 7: "M3_EWORKSPACE", 8: "M3_ELOOKBACK"}

# every symbol include/m3.h declares
EXPORTS = ["m3_prefill", "m3_prefill_workspace_size", "m3_prefill_plan", "m3_decode_carry_bytes",
           "m3_decode_state_init", "m3_decode_step", "m3_prologue", "m3_prefill_backward",
           "m3_prefill_backward_workspace_size", "m3_mixer_create", "m3_mixer_destroy", "m3_mixer_workspace_size",
           "m3_mixer_prefill", "m3_mixer_decode_step", "m3_status_string", "m3_last_error", "m3_abi_version",
           "m3_prefill_noalloc", "m3_noalloc_scratch_bytes", "m3_prefill_check", "m3_decode_step_fused",
           "m3_prefill_fused"]


class M3Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("heads", ctypes.c_int32),
                ("groups", ctypes.c_int32), ("headdim", ctypes.c_int32), ("dstate", ctypes.c_int32)]


class M3Plan(ctypes.Structure):
    _fields_ = [("n_chunks", ctypes.c_int64), ("last_chunk_len", ctypes.c_int64),
                ("segments", ctypes.c_int32), ("chunks_per_segment", ctypes.c_int64),
                ("path", ctypes.c_int32), ("workspace_bytes", ctypes.c_size_t)]


class M3DecodeState(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("carry_B", ctypes.c_void_p), ("carry_x", ctypes.c_void_p),
                ("t", ctypes.c_int64), ("dims", M3Dims), ("R", ctypes.c_int32), ("io_dtype", ctypes.c_int)]


class M3MixerWeights(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32)] + [(n, ctypes.c_void_p) for n in (
        "W_x", "W_z", "W_B", "W_C", "W_dt", "W_lambda", "W_out", "B_weight", "B_bias", "C_weight", "C_bias",
        "dt_bias", "A", "omega", "D")] + [("eps", ctypes.c_float)]


class M3Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def load(path: str = LIB_PATH):
    """Load libm3.so (no GPU needed to load it). Raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m mamba_ssm_scan_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    dims_p = ctypes.POINTER(M3Dims)
    lib.m3_prefill.argtypes = [vp] * 8 + [i32, i32, vp, vp, vp, dims_p, ctypes.c_int, vp, vp, vp, sz, vp]
    lib.m3_prefill.restype = ctypes.c_int
    lib.m3_prefill_fused.argtypes = [vp] * 9 + [i32, i32, vp, vp, vp, dims_p, ctypes.c_int, vp, vp, vp, sz, vp]
    lib.m3_prefill_fused.restype = ctypes.c_int
    lib.m3_prefill_noalloc.argtypes = [vp] * 8 + [i32, i32, vp, vp, vp, dims_p, ctypes.c_int, vp, vp, vp]
    lib.m3_prefill_noalloc.restype = ctypes.c_int
    lib.m3_prefill_check.argtypes = [dims_p, i32, i32, ctypes.c_int, vp, sz, vp]
    lib.m3_prefill_check.restype = ctypes.c_int
    lib.m3_noalloc_scratch_bytes.argtypes = []
    lib.m3_noalloc_scratch_bytes.restype = sz
    lib.m3_prefill_workspace_size.argtypes = [dims_p, i32, i32, ctypes.c_int]
    lib.m3_prefill_workspace_size.restype = sz
    lib.m3_prefill_plan.argtypes = [dims_p, i32, i32, ctypes.c_int, ctypes.POINTER(M3Plan)]
    lib.m3_prefill_plan.restype = ctypes.c_int
    lib.m3_decode_carry_bytes.argtypes = [dims_p, i32, ctypes.c_int, i32]
    lib.m3_decode_carry_bytes.restype = sz
    lib.m3_decode_state_init.argtypes = [ctypes.POINTER(M3DecodeState), dims_p, i32, ctypes.c_int,
                                         vp, vp, vp, vp, vp, vp, i64, vp]
    lib.m3_decode_state_init.restype = ctypes.c_int
    lib.m3_decode_step.argtypes = [ctypes.POINTER(M3DecodeState)] + [vp] * 8 + [i32, vp, vp]
    lib.m3_decode_step.restype = ctypes.c_int
    lib.m3_decode_step_fused.argtypes = ([ctypes.POINTER(M3DecodeState)] + [vp] * 12 + [ctypes.c_float, vp, i32, vp,
                                                                                       vp])
    lib.m3_decode_step_fused.restype = ctypes.c_int
    lib.m3_prologue.argtypes = [dims_p, i32, ctypes.c_int, i64] + [vp] * 6 + [ctypes.c_float] + [vp] * 7 + [vp]
    lib.m3_prologue.restype = ctypes.c_int
    lib.m3_prefill_backward.argtypes = [vp] * 8 + [i32] + [vp] * 16 + [dims_p, ctypes.c_int, vp, sz, vp]
    lib.m3_prefill_backward.restype = ctypes.c_int
    lib.m3_prefill_backward_workspace_size.argtypes = [dims_p, i32]
    lib.m3_prefill_backward_workspace_size.restype = sz
    lib.m3_mixer_create.argtypes = [ctypes.POINTER(vp)]
    lib.m3_mixer_create.restype = ctypes.c_int
    lib.m3_mixer_destroy.argtypes = [vp]
    lib.m3_mixer_destroy.restype = None
    lib.m3_mixer_workspace_size.argtypes = [dims_p, i32, i32, i32]
    lib.m3_mixer_workspace_size.restype = sz
    lib.m3_mixer_prefill.argtypes = [vp, ctypes.POINTER(M3MixerWeights), dims_p, i32, i32, vp, vp, vp, vp,
                                     ctypes.POINTER(M3DecodeState), vp, sz, vp]
    lib.m3_mixer_prefill.restype = ctypes.c_int
    lib.m3_mixer_decode_step.argtypes = [vp, ctypes.POINTER(M3MixerWeights), ctypes.POINTER(M3DecodeState), vp, vp,
                                         vp, sz, vp]
    lib.m3_mixer_decode_step.restype = ctypes.c_int
    lib.m3_status_string.argtypes = [ctypes.c_int]
    lib.m3_status_string.restype = ctypes.c_char_p
    lib.m3_last_error.argtypes = []
    lib.m3_last_error.restype = ctypes.c_char_p
    lib.m3_abi_version.argtypes = []
    lib.m3_abi_version.restype = i32
    _lib = lib
    return lib


def check(status: int):
    if status != 0:
        raise M3Error(status, load().m3_last_error().decode())


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return M3_BF16
    if dtype == torch.float32:
        return M3_F32
    raise TypeError(f"io dtype must be bfloat16 or float32, got {dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], name: str, dtype: Optional[torch.dtype] = None, shape=None):
    """Check a tensor argument; return it, or an aligned copy if its data is not 16-byte aligned."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.data_ptr() % 16:
        t = t.clone()
    return t


def _need_out(t, name, dtype, shape):
    """Outputs are written in place, so they must already be aligned."""
    if t is None:
        return
    if _need(t, name, dtype, shape) is not t:
        raise ValueError(f"{name} must be 16-byte aligned")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dims(batch, seqlen, heads, groups, headdim, dstate) -> M3Dims:
    return M3Dims(batch, seqlen, heads, groups, headdim, dstate)


def plan(d: M3Dims, R: int, chunk: int, io_dtype: int) -> M3Plan:
    p = M3Plan()
    check(load().m3_prefill_plan(ctypes.byref(d), R, chunk, io_dtype, ctypes.byref(p)))
    return p


def prefill(x, dt, A, omega, lam, B, C, D, R: int, chunk: int, h0=None, *, carry_B=None, carry_x=None,
            y=None, h_out=None, workspace=None, return_state: bool = True, stream=None, raw_steps: bool = False,
            dt_bias=None):
    """m3_prefill on torch device tensors; returns (y, h_out).

    x [b][L][H][R][P], B/C [b][L][G][R][N] (bf16 or fp32, one dtype), dt/lam
    [b][L][H] fp32, A/D [H], omega [H][N/2], h0 [b][H][N][P] fp32 or None.
    raw_steps: m3_prefill_fused -- dt and lam are raw projections (softplus with
    dt_bias [H] or None, sigmoid).
    """
    if x.dim() != 5 or B.dim() != 5:
        raise ValueError("x must be [b][L][H][R][P] and B [b][L][G][R][N]")
    b, L, H, R_, P = x.shape
    G, N = B.shape[2], B.shape[4]
    if R_ != R or B.shape[3] != R:
        raise ValueError(f"rank mismatch: R={R}, x has {R_}, B has {B.shape[3]}")
    io = x.dtype
    x = _need(x, "x", io)
    B = _need(B, "B", io, (b, L, G, R, N))
    C = _need(C, "C", io, (b, L, G, R, N))
    dt = _need(dt, "dt", torch.float32, (b, L, H))
    lam = _need(lam, "lambda", torch.float32, (b, L, H))
    A = _need(A, "A", torch.float32, (H,))
    D = _need(D, "D", torch.float32, (H,))
    omega = _need(omega, "omega", torch.float32, (H, N // 2))
    h0 = _need(h0, "h0", torch.float32, (b, H, N, P))
    carry_B = _need(carry_B, "carry_B", io, (b, G, R, N))
    carry_x = _need(carry_x, "carry_x", io, (b, H, R, P))
    dt_bias = _need(dt_bias, "dt_bias", torch.float32, (H,))
    if dt_bias is not None and not raw_steps:
        raise ValueError("dt_bias is only read with raw_steps")
    if y is None:
        y = torch.empty_like(x)
    _need_out(y, "y", io, x.shape)
    if h_out is None and return_state:
        h_out = torch.empty((b, H, N, P), dtype=torch.float32, device=x.device)
    _need_out(h_out, "h_out", torch.float32, (b, H, N, P))
    d = dims(b, L, H, G, P, N)
    code = _io_code(io)
    lib = load()
    need = lib.m3_prefill_workspace_size(ctypes.byref(d), R, chunk, code)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if raw_steps:
        check(lib.m3_prefill_fused(_ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(omega), _ptr(lam), _ptr(B),
                                   _ptr(C), _ptr(D), R, chunk, _ptr(h0), _ptr(y), _ptr(h_out), ctypes.byref(d), code,
                                   _ptr(carry_B), _ptr(carry_x), _ptr(workspace), ws_bytes, _stream(stream)))
        return y, h_out
    check(lib.m3_prefill(_ptr(x), _ptr(dt), _ptr(A), _ptr(omega), _ptr(lam), _ptr(B), _ptr(C), _ptr(D),
                         R, chunk, _ptr(h0), _ptr(y), _ptr(h_out), ctypes.byref(d), code,
                         _ptr(carry_B), _ptr(carry_x), _ptr(workspace), ws_bytes, _stream(stream)))
    return y, h_out


class DecodeState:
    """Caller-owned decode state: fp32 h plus the carry (the previous token's B rows per group and x rows per
    head), bound to libm3."""

    def __init__(self, batch, heads, groups, headdim, dstate, R, io_dtype=torch.bfloat16, device="cuda",
                 h0=None, B_last=None, x_last=None, t0: int = 0, stream=None):
        self.dims = dims(batch, 1, heads, groups, headdim, dstate)
        self.R = R
        self.io_dtype = io_dtype
        self.h = torch.empty((batch, heads, dstate, headdim), dtype=torch.float32, device=device)
        # carry_B is opaque: two slots of the group's previous B rows and a parity word per head
        nB = load().m3_decode_carry_bytes(ctypes.byref(self.dims), R, _io_code(io_dtype), 0)
        if nB == 0 and batch > 0:
            raise M3Error(1, "invalid decode state sizes")
        self.carry_B = torch.empty((max(nB, 16),), dtype=torch.uint8, device=device)
        self.carry_x = torch.empty((batch, heads, R, headdim), dtype=io_dtype, device=device)
        h0 = _need(h0, "h0", torch.float32, self.h.shape)
        B_last = _need(B_last, "B_last", io_dtype, (batch, groups, R, dstate))
        x_last = _need(x_last, "x_last", io_dtype, (batch, heads, R, headdim))
        self._st = M3DecodeState()
        check(load().m3_decode_state_init(ctypes.byref(self._st), ctypes.byref(self.dims), R, _io_code(io_dtype),
                                          _ptr(self.h), _ptr(self.carry_B), _ptr(self.carry_x), _ptr(h0),
                                          _ptr(B_last), _ptr(x_last), t0, _stream(stream)))
        self._keep = (h0, B_last, x_last)

    @property
    def t(self) -> int:
        return int(self._st.t)

    def step(self, x_t, dt_t, A, omega, lam_t, B_t, C_t, D, y_t=None, stream=None):
        """m3_decode_step: one token for every (b, h); returns y_t [b][H][R][P]."""
        b, H, G = self.dims.batch, self.dims.heads, self.dims.groups
        P, N, R = self.dims.headdim, self.dims.dstate, self.R
        x_t = _need(x_t, "x_t", self.io_dtype, (b, H, R, P))
        B_t = _need(B_t, "B_t", self.io_dtype, (b, G, R, N))
        C_t = _need(C_t, "C_t", self.io_dtype, (b, G, R, N))
        dt_t = _need(dt_t, "dt_t", torch.float32, (b, H))
        lam_t = _need(lam_t, "lambda_t", torch.float32, (b, H))
        A = _need(A, "A", torch.float32, (H,))
        D = _need(D, "D", torch.float32, (H,))
        omega = _need(omega, "omega", torch.float32, (H, N // 2))
        if y_t is None:
            y_t = torch.empty_like(x_t)
        _need_out(y_t, "y_t", self.io_dtype, x_t.shape)
        check(load().m3_decode_step(ctypes.byref(self._st), _ptr(x_t), _ptr(dt_t), _ptr(A), _ptr(omega),
                                    _ptr(lam_t), _ptr(B_t), _ptr(C_t), _ptr(D), R, _ptr(y_t), _stream(stream)))
        return y_t

    def step_fused(self, x_t, dt_raw_t, A, omega, lambda_raw_t, B_raw_t, C_raw_t, D, *, dt_bias=None, B_weight=None,
                   B_bias=None, C_weight=None, C_bias=None, eps: float = 1e-6, y_t=None, stream=None):
        """m3_decode_step_fused: one token from the raw projections (norm, weight and bias on B_t and C_t,
        softplus on dt_raw_t + dt_bias, sigmoid on lambda_raw_t) in the step kernel; returns y_t."""
        b, H, G = self.dims.batch, self.dims.heads, self.dims.groups
        P, N, R = self.dims.headdim, self.dims.dstate, self.R
        x_t = _need(x_t, "x_t", self.io_dtype, (b, H, R, P))
        B_raw_t = _need(B_raw_t, "B_raw_t", self.io_dtype, (b, G, R, N))
        C_raw_t = _need(C_raw_t, "C_raw_t", self.io_dtype, (b, G, R, N))
        dt_raw_t = _need(dt_raw_t, "dt_raw_t", torch.float32, (b, H))
        lambda_raw_t = _need(lambda_raw_t, "lambda_raw_t", torch.float32, (b, H))
        A = _need(A, "A", torch.float32, (H,))
        D = _need(D, "D", torch.float32, (H,))
        omega = _need(omega, "omega", torch.float32, (H, N // 2))
        dt_bias = _need(dt_bias, "dt_bias", torch.float32, (H,))
        w = [_need(v, n, torch.float32, (G, R, N)) for v, n in
             ((B_weight, "B_weight"), (B_bias, "B_bias"), (C_weight, "C_weight"), (C_bias, "C_bias"))]
        if y_t is None:
            y_t = torch.empty_like(x_t)
        _need_out(y_t, "y_t", self.io_dtype, x_t.shape)
        check(load().m3_decode_step_fused(ctypes.byref(self._st), _ptr(x_t), _ptr(dt_raw_t), _ptr(dt_bias), _ptr(A),
                                          _ptr(omega), _ptr(lambda_raw_t), _ptr(B_raw_t), _ptr(C_raw_t),
                                          *[_ptr(v) for v in w], float(eps), _ptr(D), R, _ptr(y_t),
                                          _stream(stream)))
        return y_t

    def step_raw(self, x_t, dt_t, A, omega, lam_t, B_t, C_t, D, y_t, stream_handle: ctypes.c_void_p):
        """The same call with no checks on the Python side (shapes were checked once by the caller)."""
        check(_lib.m3_decode_step(ctypes.byref(self._st), ctypes.c_void_p(x_t), ctypes.c_void_p(dt_t),
                                  ctypes.c_void_p(A), ctypes.c_void_p(omega), ctypes.c_void_p(lam_t),
                                  ctypes.c_void_p(B_t), ctypes.c_void_p(C_t), ctypes.c_void_p(D), self.R,
                                  ctypes.c_void_p(y_t), stream_handle))


def prologue(B_raw=None, C_raw=None, *, B_weight=None, B_bias=None, C_weight=None, C_bias=None, eps: float = 1e-6,
             dt_raw=None, dt_bias=None, lambda_raw=None, heads: Optional[int] = None,
             B=None, C=None, dt=None, lam=None, stream=None):
    """m3_prologue on torch device tensors; returns (B, C, dt, lambda), None for parts not given.

    B_raw, C_raw [..., G, R, N] (bf16 or fp32, one dtype); B/C weights and biases
    [G, R, N] fp32; dt_raw, lambda_raw [..., H] fp32 with the same leading axes
    (the token axes); dt_bias [H]. Outputs are allocated unless given (an output
    may be its own input: in place).
    """
    rows = B_raw if B_raw is not None else C_raw
    scal = dt_raw if dt_raw is not None else lambda_raw
    if rows is None and scal is None:
        raise ValueError("nothing to do: give B_raw / C_raw and / or dt_raw / lambda_raw")
    if rows is not None:
        if rows.dim() < 3:
            raise ValueError("B_raw / C_raw must be [..., G, R, N]")
        G, R, N = rows.shape[-3:]
        lead = tuple(rows.shape[:-3])
        io = rows.dtype
    if scal is not None:
        H = scal.shape[-1]
        if rows is not None and tuple(scal.shape[:-1]) != lead:
            raise ValueError("dt_raw / lambda_raw token axes differ from B_raw / C_raw")
        lead = tuple(scal.shape[:-1])
    else:
        H = heads or G
    if rows is None:
        G, R, N, io = 1, 1, 2, torch.bfloat16
    ntok = 1
    for v in lead:
        ntok *= v
    B_raw = _need(B_raw, "B_raw", io, lead + (G, R, N))
    C_raw = _need(C_raw, "C_raw", io, lead + (G, R, N))
    B_weight = _need(B_weight, "B_weight", torch.float32, (G, R, N))
    B_bias = _need(B_bias, "B_bias", torch.float32, (G, R, N))
    C_weight = _need(C_weight, "C_weight", torch.float32, (G, R, N))
    C_bias = _need(C_bias, "C_bias", torch.float32, (G, R, N))
    dt_raw = _need(dt_raw, "dt_raw", torch.float32, lead + (H,))
    dt_bias = _need(dt_bias, "dt_bias", torch.float32, (H,))
    lambda_raw = _need(lambda_raw, "lambda_raw", torch.float32, lead + (H,))
    if B_raw is not None and B is None:
        B = torch.empty_like(B_raw)
    if C_raw is not None and C is None:
        C = torch.empty_like(C_raw)
    if dt_raw is not None and dt is None:
        dt = torch.empty_like(dt_raw)
    if lambda_raw is not None and lam is None:
        lam = torch.empty_like(lambda_raw)
    _need_out(B, "B", io, lead + (G, R, N))
    _need_out(C, "C", io, lead + (G, R, N))
    _need_out(dt, "dt", torch.float32, lead + (H,))
    _need_out(lam, "lambda", torch.float32, lead + (H,))
    d = dims(ntok, 1, H, G, 1, N)
    check(load().m3_prologue(ctypes.byref(d), R, _io_code(io), ntok, _ptr(B_raw), _ptr(C_raw), _ptr(B_weight),
                             _ptr(B_bias), _ptr(C_weight), _ptr(C_bias), ctypes.c_float(eps), _ptr(dt_raw),
                             _ptr(dt_bias), _ptr(lambda_raw), _ptr(B), _ptr(C), _ptr(dt), _ptr(lam),
                             _stream(stream)))
    return B, C, dt, lam


def prefill_backward(x, dt, A, omega, lam, B, C, D, R: int, dy, h0=None, dh_out=None, *, carry_B=None,
                     carry_x=None, want_lambda=True, want_omega=True, want_h0=True, workspace=None, stream=None):
    """m3_prefill_backward on torch device tensors; returns a dict of fp32 gradients.

    Keys: x, B, C, dt, lam, A, omega, D, h0, carry_B, carry_x (None for gradients
    not asked for or without a carry). Inputs as for `prefill`; dy like y.
    """
    if x.dim() != 5 or B.dim() != 5:
        raise ValueError("x must be [b][L][H][R][P] and B [b][L][G][R][N]")
    b, L, H, R_, P = x.shape
    G, N = B.shape[2], B.shape[4]
    if R_ != R or B.shape[3] != R:
        raise ValueError(f"rank mismatch: R={R}, x has {R_}, B has {B.shape[3]}")
    io = x.dtype
    x = _need(x, "x", io)
    B = _need(B, "B", io, (b, L, G, R, N))
    C = _need(C, "C", io, (b, L, G, R, N))
    dy = _need(dy, "dy", io, (b, L, H, R, P))
    dt = _need(dt, "dt", torch.float32, (b, L, H))
    lam = _need(lam, "lambda", torch.float32, (b, L, H))
    A = _need(A, "A", torch.float32, (H,))
    D = _need(D, "D", torch.float32, (H,))
    omega = _need(omega, "omega", torch.float32, (H, N // 2))
    h0 = _need(h0, "h0", torch.float32, (b, H, N, P))
    dh_out = _need(dh_out, "dh_out", torch.float32, (b, H, N, P))
    carry_B = _need(carry_B, "carry_B", io, (b, G, R, N))
    carry_x = _need(carry_x, "carry_x", io, (b, H, R, P))
    f32 = dict(dtype=torch.float32, device=x.device)
    g = {"x": torch.empty((b, L, H, R, P), **f32), "B": torch.empty((b, L, G, R, N), **f32),
         "C": torch.empty((b, L, G, R, N), **f32), "dt": torch.empty((b, L, H), **f32),
         "lam": torch.empty((b, L, H), **f32) if want_lambda else None, "A": torch.empty((H,), **f32),
         "omega": torch.empty((H, N // 2), **f32) if want_omega else None, "D": torch.empty((H,), **f32),
         "h0": torch.empty((b, H, N, P), **f32) if want_h0 else None,
         "carry_B": torch.empty((b, G, R, N), **f32) if carry_B is not None else None,
         "carry_x": torch.empty((b, H, R, P), **f32) if carry_x is not None else None}
    d = dims(b, L, H, G, P, N)
    lib = load()
    need = lib.m3_prefill_backward_workspace_size(ctypes.byref(d), R)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.m3_prefill_backward(_ptr(x), _ptr(dt), _ptr(A), _ptr(omega), _ptr(lam), _ptr(B), _ptr(C), _ptr(D),
                                  R, _ptr(h0), _ptr(carry_B), _ptr(carry_x), _ptr(dy), _ptr(dh_out),
                                  _ptr(g["x"]), _ptr(g["B"]), _ptr(g["C"]), _ptr(g["dt"]), _ptr(g["lam"]),
                                  _ptr(g["A"]), _ptr(g["omega"]), _ptr(g["D"]), _ptr(g["h0"]), _ptr(g["carry_B"]),
                                  _ptr(g["carry_x"]), ctypes.byref(d), _io_code(io), _ptr(workspace), ws_bytes,
                                  _stream(stream)))
    return g


class Mixer:
    """The mixer block (m3_mixer_*): projections, prologue, recurrence, silu gate, output projection.

    w: a dict with the bf16 weights W_x, W_z, W_B, W_C, W_dt, W_lambda [*][d_model]
    and W_out [d_model][H*R*P] (row-major [out][in], as a linear layer), fp32 B_weight, B_bias,
    C_weight, C_bias [G][R][N], dt_bias, A, D [H], omega [H][N/2] (the optional
    ones may be None), eps, and the sizes H, G, R, P, N, d_model.
    """

    def __init__(self, w: dict):
        lib = load()
        self.H, self.G, self.R, self.P, self.N, self.d_model = (int(w[k]) for k in ("H", "G", "R", "P", "N",
                                                                                    "d_model"))
        HRP, GRN, dm = self.H * self.R * self.P, self.G * self.R * self.N, self.d_model
        bf, f32 = torch.bfloat16, torch.float32
        shapes = {"W_x": (HRP, dm, bf), "W_z": (HRP, dm, bf), "W_B": (GRN, dm, bf), "W_C": (GRN, dm, bf),
                  "W_dt": (self.H, dm, bf), "W_lambda": (self.H, dm, bf), "W_out": (dm, HRP, bf)}
        keep = {k: _need(w[k], k, dt, (r, c)) for k, (r, c, dt) in shapes.items()}
        par = (self.G, self.R, self.N)
        for k in ("B_weight", "B_bias", "C_weight", "C_bias"):
            keep[k] = _need(w.get(k), k, f32, par)
        keep["dt_bias"] = _need(w.get("dt_bias"), "dt_bias", f32, (self.H,))
        keep["A"] = _need(w["A"], "A", f32, (self.H,))
        keep["D"] = _need(w["D"], "D", f32, (self.H,))
        keep["omega"] = _need(w.get("omega"), "omega", f32, (self.H, self.N // 2))
        self._keep = keep
        self._w = M3MixerWeights(dm, *[_ptr(keep[k]) for k in ("W_x", "W_z", "W_B", "W_C", "W_dt", "W_lambda",
                                                                 "W_out", "B_weight", "B_bias", "C_weight", "C_bias",
                                                                 "dt_bias", "A", "omega", "D")], float(w["eps"]))
        h = ctypes.c_void_p()
        check(lib.m3_mixer_create(ctypes.byref(h)))
        self._h = h
        self._ws = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.m3_mixer_destroy(h)
            self._h = None

    def workspace(self, batch: int, seqlen: int, chunk: int = 64) -> torch.Tensor:
        d = dims(batch, seqlen, self.H, self.G, self.P, self.N)
        n = load().m3_mixer_workspace_size(ctypes.byref(d), self.R, chunk, self.d_model)
        if n == 0:
            raise ValueError("invalid block sizes")
        key = (batch, seqlen, chunk)
        if key not in self._ws or self._ws[key].numel() < n:
            self._ws[key] = torch.empty(n, dtype=torch.uint8, device="cuda")
        return self._ws[key]

    def decode_state(self, batch: int) -> DecodeState:
        return DecodeState(batch, self.H, self.G, self.P, self.N, self.R, io_dtype=torch.bfloat16)

    def prefill(self, u, chunk: int = 64, h0=None, out=None, h_out=None, state: Optional[DecodeState] = None,
                stream=None):
        """u [b][L][d_model] bf16 -> out [b][L][d_model]; h_out [b][H][N][P] fp32 when requested (True or a tensor)."""
        b, L, dm = u.shape
        u = _need(u, "u", torch.bfloat16, (b, L, self.d_model))
        if out is None:
            out = torch.empty_like(u)
        _need_out(out, "out", torch.bfloat16, u.shape)
        hs = (b, self.H, self.N, self.P)
        h0 = _need(h0, "h0", torch.float32, hs)
        if h_out is True:
            h_out = torch.empty(hs, dtype=torch.float32, device=u.device)
        _need_out(h_out, "h_out", torch.float32, hs)
        d = dims(b, L, self.H, self.G, self.P, self.N)
        ws = self.workspace(b, L, chunk)
        st = ctypes.byref(state._st) if state is not None else None
        check(load().m3_mixer_prefill(self._h, ctypes.byref(self._w), ctypes.byref(d), self.R, chunk, _ptr(u),
                                      _ptr(out), _ptr(h0), _ptr(h_out), st, _ptr(ws), ws.numel(), _stream(stream)))
        return out, h_out

    def decode_step(self, state: DecodeState, u_t, out_t=None, stream=None):
        """u_t [b][d_model] bf16 -> out_t [b][d_model], advancing the state by one token."""
        b = state.dims.batch
        u_t = _need(u_t, "u_t", torch.bfloat16, (b, self.d_model))
        if out_t is None:
            out_t = torch.empty_like(u_t)
        _need_out(out_t, "out_t", torch.bfloat16, u_t.shape)
        ws = self.workspace(b, 1)
        check(load().m3_mixer_decode_step(self._h, ctypes.byref(self._w), ctypes.byref(state._st), _ptr(u_t),
                                          _ptr(out_t), _ptr(ws), ws.numel(), _stream(stream)))
        return out_t
