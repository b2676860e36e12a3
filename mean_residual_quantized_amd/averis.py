"""Thin ctypes binding of libaveris (include/averis.h), same names as the C ABI.

Argument marshalling only: torch supplies device memory (outputs and
workspace are allocated with torch.empty) and the current HIP stream; every
step of the computation runs in the library's kernels.  The library must be
built (``python -m mean_residual_quantized_amd.build``); if it is missing,
loading fails with an error -- there is no fallback.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libaveris.so")

AVERIS_OK = 0
STATUS_NAMES = {0: "OK", 1: "E_NULL", 2: "E_SHAPE", 3: "E_DTYPE", 4: "E_ALIGN",
                5: "E_WORKSPACE", 6: "E_ARG", 7: "E_HIP"}
F32, BF16 = 0, 1
RN, SR = 0, 1
OP_SPLIT_QUANT, OP_QUANT, OP_GEMM, OP_WGRAD, OP_QUANT_PAIR_MULTI = 0, 1, 2, 3, 4
MAX_WEIGHTS = 16
MAX_RANK1 = 4
STREAM_ACT, STREAM_MEAN, STREAM_WEIGHT, STREAM_RESIDUAL_T = 0, 1, 2, 3

# every symbol include/averis.h declares
EXPORTS = [
    "averis_split_quant", "averis_split_quant_grouped", "averis_quant", "averis_quant_batched",
    "averis_quant_grouped", "averis_quant_pair", "averis_quant_pair_2d",
    "averis_quant_pair_multi", "averis_gemm_fwd", "averis_gemm_dgrad",
    "averis_gemm_vanilla", "averis_gemm_grouped", "averis_residual_t_quant", "averis_gemm_wgrad",
    "averis_split_quant_ratio", "averis_split_quant_rank1", "averis_split_quant_rank1_multi",
    "averis_gemm_rank1",
    "averis_split_quant_grouped_rank1", "averis_gemm_grouped_rank1",
    "averis_split_quant_noalloc", "averis_gemm_rank1_stats", "averis_split_quant_from_stats",
    "averis_workspace_bytes", "averis_status_str",
    "averis_abi_version", "averis_last_error",
]


class AverisError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s failed: %s (%s)" % (fn, STATUS_NAMES.get(status, status), msg))
        self.status = status


class _NVFP4(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tscale", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class _Weight(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("lda", ctypes.c_int64), ("seed", ctypes.c_uint64),
                ("out", ctypes.POINTER(_NVFP4)), ("out_t", ctypes.POINTER(_NVFP4))]


_lib = None


def lib():
    """Load libaveris.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libaveris.so not built at %s; run "
                               "`python -m mean_residual_quantized_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, U64, I, U32, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_uint32, ctypes.c_size_t)
        T = ctypes.POINTER(_NVFP4)
        sig = {
            "averis_split_quant": [P, I, I64, I64, I64, U64, I, T, T, P, P, SZ, P],
            "averis_split_quant_grouped": [P, I, I64, I64, I64, P, I, U64, I, T, T, P, P, SZ, P],
            "averis_quant": [P, I, I64, I64, I64, I, U64, I, U32, T, P, SZ, P],
            "averis_quant_batched": [P, I, I, I64, I64, I64, I64, I, U64, I, U32, T, P, SZ, P],
            "averis_quant_grouped": [P, I, I64, I64, I64, P, I, U64, I, U32, T, P, SZ, P],
            "averis_quant_pair": [P, I, I, I64, I64, I64, I64, U64, I, U32, T, T, P, SZ, P],
            "averis_quant_pair_2d": [P, I, I, I64, I64, I64, I64, U64, I, U32, T, T, P, SZ, P],
            "averis_quant_pair_multi": [I, P, I, I, U32, P, SZ, P],
            "averis_gemm_fwd": [T, T, T, P, I, I64, P, SZ, P],
            "averis_gemm_dgrad": [T, T, T, P, I, I64, P, SZ, P],
            "averis_gemm_vanilla": [T, T, P, I, I64, P, SZ, P],
            "averis_gemm_grouped": [T, T, T, P, I, P, I, I64, P, SZ, P],
            "averis_residual_t_quant": [P, I, I64, I64, I64, P, P, U64, I, T, P],
            "averis_gemm_wgrad": [T, T, P, P, P, I, I64, P, SZ, P],
            "averis_split_quant_ratio": [P, I, I64, I64, I64, P, I, U64, I, T, T, P, P, P, SZ, P],
            "averis_split_quant_rank1": [P, I, I64, I64, I64, U64, I, T, T, P, T, P, P, SZ, P],
            "averis_gemm_rank1": [T, P, T, P, I, I64, P],
            "averis_split_quant_rank1_multi": [P, I, I64, I64, I64, U64, I, T, T, P, I, P, P, P,
                                               SZ, P],
            "averis_split_quant_grouped_rank1": [P, I, I64, I64, I64, P, I, U64, I, T, T, P, T, P,
                                                 P, SZ, P],
            "averis_gemm_grouped_rank1": [T, P, T, P, I, P, I, I64, P],
            "averis_split_quant_noalloc": [P, I, I64, I64, I64, U64, I, T, T, P, P],
            "averis_gemm_rank1_stats": [T, P, T, P, I64, P, SZ, P],
            "averis_split_quant_from_stats": [P, I64, I64, I64, U64, I, T, T, P, T, P, P, SZ, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.averis_workspace_bytes.argtypes = [I, I64, I64, I64, I64]
        L.averis_workspace_bytes.restype = SZ
        L.averis_status_str.argtypes = [I]
        L.averis_status_str.restype = ctypes.c_char_p
        L.averis_abi_version.argtypes = []
        L.averis_abi_version.restype = I
        L.averis_last_error.argtypes = []
        L.averis_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn, status):
    if status != AVERIS_OK:
        msg = lib().averis_status_str(status).decode()
        if status == 7:
            msg += ": " + lib().averis_last_error().decode()
        raise AverisError(fn, status, msg)


def workspace_bytes(op, rows, cols, n=0, nseg=0):
    return int(lib().averis_workspace_bytes(op, rows, cols, n, nseg))


# --------------------------------------------------------------------------
# tensors
# --------------------------------------------------------------------------

@dataclass
class NVFP4:
    """Device NVFP4-style tensor: codes u8[rows, cols/2], scales u8[rows, cols/16]
    (E4M3), tscale f32[2*nseg] = [S_enc, S_dec] per segment."""
    codes: torch.Tensor
    scales: torch.Tensor
    tscale: torch.Tensor
    rows: int
    cols: int

    @staticmethod
    def empty(rows, cols, nseg=1, device="cuda"):
        return NVFP4(torch.empty((rows, cols // 2), dtype=torch.uint8, device=device),
                     torch.empty((rows, cols // 16), dtype=torch.uint8, device=device),
                     torch.empty((2 * nseg,), dtype=torch.float32, device=device), rows, cols)

    def c(self):
        return _NVFP4(self.codes.data_ptr(), self.scales.data_ptr(), self.tscale.data_ptr(),
                      self.rows, self.cols)

    def cpu(self):
        return dict(codes=self.codes.cpu().numpy(), scales=self.scales.cpu().numpy(),
                    tscale=self.tscale.cpu().numpy())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("libaveris takes float32 or bfloat16 inputs, got %s" % t.dtype)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _workspace(nbytes, device):
    return torch.empty((max(int(nbytes), 1),), dtype=torch.uint8, device=device)


def _lda(a):
    if a.dim() != 2 or a.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return a.stride(0)


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def averis_split_quant(a, seed=0, rnd=SR, ws=None):
    """Q4(a - 1 mu) and Q4(mu); returns (residual, mean, mu_f32)."""
    rows, cols = a.shape
    res = NVFP4.empty(rows, cols, 1, a.device)
    mean = NVFP4.empty(1, cols, 1, a.device)
    mu = torch.empty((cols,), dtype=torch.float32, device=a.device)
    need = workspace_bytes(OP_SPLIT_QUANT, rows, cols)
    ws = ws if ws is not None else _workspace(need, a.device)
    r, m = res.c(), mean.c()
    _check("averis_split_quant", lib().averis_split_quant(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), seed, rnd, ctypes.byref(r),
        ctypes.byref(m), mu.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return res, mean, mu


def averis_split_quant_noalloc(a, seed=0, rnd=SR):
    """averis_split_quant with the library's own device array as the
    workspace (no workspace argument); returns (residual, mean, mu_f32)."""
    rows, cols = a.shape
    res = NVFP4.empty(rows, cols, 1, a.device)
    mean = NVFP4.empty(1, cols, 1, a.device)
    mu = torch.empty((cols,), dtype=torch.float32, device=a.device)
    r, m = res.c(), mean.c()
    _check("averis_split_quant_noalloc", lib().averis_split_quant_noalloc(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), seed, rnd, ctypes.byref(r),
        ctypes.byref(m), mu.data_ptr(), _stream()))
    return res, mean, mu


def averis_split_quant_grouped(a, offsets, seed=0, rnd=SR, ws=None):
    """Per-segment split-quant; offsets: int64 device tensor [nseg+1]."""
    rows, cols = a.shape
    nseg = offsets.numel() - 1
    res = NVFP4.empty(rows, cols, nseg, a.device)
    mean = NVFP4.empty(nseg, cols, nseg, a.device)
    mu = torch.empty((nseg, cols), dtype=torch.float32, device=a.device)
    need = workspace_bytes(OP_SPLIT_QUANT, rows, cols, 0, nseg)
    ws = ws if ws is not None else _workspace(need, a.device)
    r, m = res.c(), mean.c()
    _check("averis_split_quant_grouped", lib().averis_split_quant_grouped(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), offsets.data_ptr(), nseg, seed, rnd,
        ctypes.byref(r), ctypes.byref(m), mu.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return res, mean, mu


def averis_quant(a, transpose=False, seed=0, rnd=SR, sr_stream=STREAM_ACT, ws=None, out=None):
    """Plain Q4.  transpose=True quantizes a^T (blocks along a's rows).  out:
    an NVFP4 of the output's shape to write into (else a new one)."""
    srows, scols = a.shape
    rows, cols = (scols, srows) if transpose else (srows, scols)
    out = out if out is not None else NVFP4.empty(rows, cols, 1, a.device)
    need = workspace_bytes(OP_QUANT, rows, cols)
    ws = ws if ws is not None else _workspace(need, a.device)
    o = out.c()
    _check("averis_quant", lib().averis_quant(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), int(transpose), seed, rnd, sr_stream,
        ctypes.byref(o), ws.data_ptr(), ws.numel(), _stream()))
    return out


def averis_quant_batched(a, transpose=False, seed=0, rnd=RN, sr_stream=STREAM_WEIGHT, ws=None):
    """Plain Q4 of each matrix a[b] (3-D tensor), one tensor scale each."""
    batch, srows, scols = a.shape
    if a.stride(2) != 1:
        raise ValueError("expected unit innermost stride")
    rows, cols = (scols, srows) if transpose else (srows, scols)
    out = NVFP4.empty(batch * rows, cols, batch, a.device)
    need = workspace_bytes(OP_QUANT, rows, cols, 0, batch)
    ws = ws if ws is not None else _workspace(need, a.device)
    o = out.c()
    _check("averis_quant_batched", lib().averis_quant_batched(
        a.data_ptr(), _dtype_code(a), batch, rows, cols, a.stride(1), a.stride(0),
        int(transpose), seed, rnd, sr_stream, ctypes.byref(o), ws.data_ptr(), ws.numel(),
        _stream()))
    return out


def averis_quant_pair(w, seed=0, rnd=RN, sr_stream=STREAM_WEIGHT, ws=None):
    """Both quantized copies of a weight in one call: returns (wt, wd) with
    wt = Q4(w^T) (blocks along w's rows; the forward operand) and wd = Q4(w)
    (blocks along w's cols; the dgrad operand).  w: 2-D, or 3-D (batch of
    matrices, one tensor scale each)."""
    a = w if w.dim() == 3 else w.unsqueeze(0)
    batch, rows, cols = a.shape
    if a.stride(2) != 1:
        raise ValueError("expected unit innermost stride")
    wd = NVFP4.empty(batch * rows, cols, batch, w.device)
    wt = NVFP4.empty(batch * cols, rows, batch, w.device)
    need = workspace_bytes(OP_QUANT, rows, cols, 0, batch)
    ws = ws if ws is not None else _workspace(need, w.device)
    o, ot = wd.c(), wt.c()
    _check("averis_quant_pair", lib().averis_quant_pair(
        a.data_ptr(), _dtype_code(a), batch, rows, cols, a.stride(1), a.stride(0), seed, rnd,
        sr_stream, ctypes.byref(o), ctypes.byref(ot), ws.data_ptr(), ws.numel(), _stream()))
    return wt, wd


def averis_quant_pair_multi(ws_list, seeds=None, rnd=RN, sr_stream=STREAM_WEIGHT, ws=None):
    """Both quantized copies of several 2-D weights (one dtype, shapes of their
    own) in two launches: returns [(wt, wd), ...] in order, each as
    averis_quant_pair(w, seed) returns it."""
    n = len(ws_list)
    if not 1 <= n <= MAX_WEIGHTS:
        raise ValueError("expected 1 .. %d weights" % MAX_WEIGHTS)
    seeds = [0] * n if seeds is None else list(seeds)
    dev = ws_list[0].device
    dt = _dtype_code(ws_list[0])
    outs, keep = [], []
    arr = (_Weight * n)()
    for i, w in enumerate(ws_list):
        if w.dim() != 2 or w.stride(1) != 1:
            raise ValueError("expected 2-D weights with unit innermost stride")
        if _dtype_code(w) != dt:
            raise ValueError("expected weights of one dtype")
        rows, cols = w.shape
        wd = NVFP4.empty(rows, cols, 1, dev)
        wt = NVFP4.empty(cols, rows, 1, dev)
        o, ot = wd.c(), wt.c()
        keep += [o, ot]
        arr[i] = _Weight(w.data_ptr(), rows, cols, w.stride(0), seeds[i],
                         ctypes.pointer(o), ctypes.pointer(ot))
        outs.append((wt, wd))
    need = workspace_bytes(OP_QUANT_PAIR_MULTI, 0, 0, n)
    ws = ws if ws is not None else _workspace(need, dev)
    _check("averis_quant_pair_multi", lib().averis_quant_pair_multi(
        n, ctypes.cast(arr, ctypes.c_void_p), dt, rnd, sr_stream, ws.data_ptr(), ws.numel(),
        _stream()))
    return outs


def averis_quant_pair_2d(w, seed=0, rnd=RN, sr_stream=STREAM_WEIGHT, ws=None):
    """Both GEMM copies of a weight from one quantization in 16 x 16 tiles:
    returns (wt, wd) as averis_quant_pair does, with deq(wt) = deq(wd)^T."""
    a = w if w.dim() == 3 else w.unsqueeze(0)
    batch, rows, cols = a.shape
    if a.stride(2) != 1:
        raise ValueError("expected unit innermost stride")
    wd = NVFP4.empty(batch * rows, cols, batch, w.device)
    wt = NVFP4.empty(batch * cols, rows, batch, w.device)
    need = workspace_bytes(OP_QUANT, rows, cols, 0, batch)
    ws = ws if ws is not None else _workspace(need, w.device)
    o, ot = wd.c(), wt.c()
    _check("averis_quant_pair_2d", lib().averis_quant_pair_2d(
        a.data_ptr(), _dtype_code(a), batch, rows, cols, a.stride(1), a.stride(0), seed, rnd,
        sr_stream, ctypes.byref(o), ctypes.byref(ot), ws.data_ptr(), ws.numel(), _stream()))
    return wt, wd


def averis_quant_grouped(a, offsets, seed=0, rnd=SR, sr_stream=STREAM_ACT, ws=None, out=None):
    """Grouped plain Q4, one tensor scale per segment.  out: an NVFP4 of the
    output's shape (nseg tensor scales) to write into (else a new one)."""
    rows, cols = a.shape
    nseg = offsets.numel() - 1
    out = out if out is not None else NVFP4.empty(rows, cols, nseg, a.device)
    need = workspace_bytes(OP_QUANT, rows, cols, 0, nseg)
    ws = ws if ws is not None else _workspace(need, a.device)
    o = out.c()
    _check("averis_quant_grouped", lib().averis_quant_grouped(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), offsets.data_ptr(), nseg, seed, rnd,
        sr_stream, ctypes.byref(o), ws.data_ptr(), ws.numel(), _stream()))
    return out


def _out(m, n, dtype, device, out):
    if out is not None:
        return out
    return torch.empty((m, n), dtype=dtype, device=device)


def _gemm(fn, a, mean, b, out_dtype, out, nseg=1, offsets=None, ws=None):
    m, k = a.rows, a.cols
    n = b.rows // (nseg if offsets is not None else 1)
    c = _out(m, n, out_dtype, a.codes.device, out)
    need = workspace_bytes(OP_GEMM, m, k, n, nseg if offsets is not None else 0)
    ws = ws if ws is not None else _workspace(need, a.codes.device)
    ca, cb = a.c(), b.c()
    cm = mean.c() if mean is not None else None
    pm = ctypes.byref(cm) if cm is not None else None
    cd = _dtype_code(c)
    if fn == "averis_gemm_vanilla":
        st = lib().averis_gemm_vanilla(ctypes.byref(ca), ctypes.byref(cb), c.data_ptr(), cd,
                                       c.stride(0), ws.data_ptr(), ws.numel(), _stream())
    elif fn == "averis_gemm_grouped":
        st = lib().averis_gemm_grouped(ctypes.byref(ca), pm, ctypes.byref(cb),
                                       offsets.data_ptr(), nseg, c.data_ptr(), cd, c.stride(0),
                                       ws.data_ptr(), ws.numel(), _stream())
    else:
        st = getattr(lib(), fn)(ctypes.byref(ca), pm, ctypes.byref(cb), c.data_ptr(), cd,
                                c.stride(0), ws.data_ptr(), ws.numel(), _stream())
    _check(fn, st)
    return c


def averis_gemm_fwd(xr, mean, wt, out_dtype=torch.float32, out=None, ws=None):
    """Y = 1 (mean W) + X_R W with wt = Q4(W^T) (n x m)."""
    return _gemm("averis_gemm_fwd", xr, mean, wt, out_dtype, out, ws=ws)


def averis_gemm_dgrad(dr, mean_d, w, out_dtype=torch.float32, out=None, ws=None):
    """dX = 1 (mean_D W^T) + D_R W^T with w = Q4(W) (m x n)."""
    return _gemm("averis_gemm_dgrad", dr, mean_d, w, out_dtype, out, ws=ws)


def averis_gemm_vanilla(a, b, out_dtype=torch.float32, out=None, ws=None):
    return _gemm("averis_gemm_vanilla", a, None, b, out_dtype, out, ws=ws)


def averis_gemm_grouped(a, mean, b, offsets, out_dtype=torch.float32, out=None, ws=None):
    nseg = offsets.numel() - 1
    return _gemm("averis_gemm_grouped", a, mean, b, out_dtype, out, nseg=nseg, offsets=offsets,
                 ws=ws)


def averis_residual_t_quant(a, mu, residual, seed=0, rnd=SR, out=None):
    """Q4((a - 1 mu)^T) (cols x rows, blocks along the tokens, SR stream 3);
    mu and residual are the fp32 mean and the residual tensor
    averis_split_quant returned for the same a."""
    rows, cols = a.shape
    out = out if out is not None else NVFP4.empty(cols, rows, 1, a.device)
    o = out.c()
    _check("averis_residual_t_quant", lib().averis_residual_t_quant(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), mu.data_ptr(),
        residual.tscale.data_ptr(), seed, rnd, ctypes.byref(o), _stream()))
    return out


def averis_gemm_wgrad(xt, dt, mu_x, mu_d, out_dtype=torch.float32, out=None, ws=None):
    """dW = deq(xt) deq(dt)^T + l mu_x mu_d^T (m x n) from the transposed
    residuals xt (m x l) and dt (n x l) and the fp32 means."""
    m, n, l = xt.rows, dt.rows, xt.cols
    c = _out(m, n, out_dtype, xt.codes.device, out)
    need = workspace_bytes(OP_WGRAD, m, l, n)
    ws = ws if ws is not None else _workspace(need, xt.codes.device)
    cx, cd = xt.c(), dt.c()
    _check("averis_gemm_wgrad", lib().averis_gemm_wgrad(
        ctypes.byref(cx), ctypes.byref(cd), mu_x.data_ptr(), mu_d.data_ptr(), c.data_ptr(),
        _dtype_code(c), c.stride(0), ws.data_ptr(), ws.numel(), _stream()))
    return c


def averis_split_quant_ratio(a, seed=0, rnd=SR, offsets=None, ws=None):
    """averis_split_quant (or its grouped form with offsets) plus the
    mean-energy ratio of each segment; returns (residual, mean, mu_f32, ratio)."""
    rows, cols = a.shape
    nseg = 1 if offsets is None else offsets.numel() - 1
    res = NVFP4.empty(rows, cols, nseg, a.device)
    mean = NVFP4.empty(nseg, cols, nseg, a.device)
    mu = torch.empty((nseg, cols) if offsets is not None else (cols,), dtype=torch.float32,
                     device=a.device)
    ratio = torch.empty((nseg,), dtype=torch.float32, device=a.device)
    need = workspace_bytes(OP_SPLIT_QUANT, rows, cols, 0, 0 if offsets is None else nseg)
    ws = ws if ws is not None else _workspace(need, a.device)
    r, m = res.c(), mean.c()
    _check("averis_split_quant_ratio", lib().averis_split_quant_ratio(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a),
        offsets.data_ptr() if offsets is not None else None, nseg, seed, rnd, ctypes.byref(r),
        ctypes.byref(m), mu.data_ptr(), ratio.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return res, mean, mu, ratio


def averis_split_quant_rank1(a, b, seed=0, rnd=SR, ws=None, rho=None, out=None):
    """averis_split_quant plus the rank-one row rho = deq(mean) deq(b)^T for
    the GEMM's B operand b; returns (residual, mean, mu_f32, rho).  out:
    (residual, mean, mu_f32) to write into (else new ones)."""
    rows, cols = a.shape
    if out is not None:
        res, mean, mu = out
    else:
        res = NVFP4.empty(rows, cols, 1, a.device)
        mean = NVFP4.empty(1, cols, 1, a.device)
        mu = torch.empty((cols,), dtype=torch.float32, device=a.device)
    rho = rho if rho is not None else torch.empty((b.rows,), dtype=torch.float32, device=a.device)
    need = workspace_bytes(OP_SPLIT_QUANT, rows, cols)
    ws = ws if ws is not None else _workspace(need, a.device)
    r, m, cb = res.c(), mean.c(), b.c()
    _check("averis_split_quant_rank1", lib().averis_split_quant_rank1(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), seed, rnd, ctypes.byref(r),
        ctypes.byref(m), mu.data_ptr(), ctypes.byref(cb), rho.data_ptr(), ws.data_ptr(),
        ws.numel(), _stream()))
    return res, mean, mu, rho


def averis_split_quant_rank1_multi(a, bs, seed=0, rnd=SR, ws=None, rhos=None):
    """averis_split_quant plus the rank-one rows of several GEMMs that take
    the split (B operands bs, at most MAX_RANK1); returns (residual, mean,
    mu_f32, [rho per operand])."""
    nb = len(bs)
    if not 1 <= nb <= MAX_RANK1:
        raise ValueError("expected 1 .. %d B operands" % MAX_RANK1)
    rows, cols = a.shape
    res = NVFP4.empty(rows, cols, 1, a.device)
    mean = NVFP4.empty(1, cols, 1, a.device)
    mu = torch.empty((cols,), dtype=torch.float32, device=a.device)
    rhos = list(rhos) if rhos is not None else [
        torch.empty((b.rows,), dtype=torch.float32, device=a.device) for b in bs]
    need = workspace_bytes(OP_SPLIT_QUANT, rows, cols)
    ws = ws if ws is not None else _workspace(need, a.device)
    r, m = res.c(), mean.c()
    cbs = [b.c() for b in bs]
    barr = (ctypes.POINTER(_NVFP4) * nb)(*[ctypes.pointer(cb) for cb in cbs])
    rarr = (ctypes.c_void_p * nb)(*[rho.data_ptr() for rho in rhos])
    _check("averis_split_quant_rank1_multi", lib().averis_split_quant_rank1_multi(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), seed, rnd, ctypes.byref(r),
        ctypes.byref(m), mu.data_ptr(), nb, ctypes.cast(barr, ctypes.c_void_p),
        ctypes.cast(rarr, ctypes.c_void_p), ws.data_ptr(), ws.numel(), _stream()))
    return res, mean, mu, rhos


def averis_gemm_rank1(a, rho, b, out_dtype=torch.float32, out=None):
    """c = deq(a) deq(b)^T + 1 rho^T."""
    c = _out(a.rows, b.rows, out_dtype, a.codes.device, out)
    ca, cb = a.c(), b.c()
    _check("averis_gemm_rank1", lib().averis_gemm_rank1(
        ctypes.byref(ca), rho.data_ptr(), ctypes.byref(cb), c.data_ptr(), _dtype_code(c),
        c.stride(0), _stream()))
    return c


def averis_split_quant_grouped_rank1(a, offsets, b, seed=0, rnd=SR, ws=None, out=None, rho=None):
    """Grouped split-quant plus rho[s] = deq(mean_s) deq(b_s)^T per segment
    (b: nseg stacked matrices); returns (residual, mean, mu_f32, rho).  out:
    (residual, mean, mu_f32) and rho: buffers to write into (else new ones)."""
    rows, cols = a.shape
    nseg = offsets.numel() - 1
    if out is not None:
        res, mean, mu = out
    else:
        res = NVFP4.empty(rows, cols, nseg, a.device)
        mean = NVFP4.empty(nseg, cols, nseg, a.device)
        mu = torch.empty((nseg, cols), dtype=torch.float32, device=a.device)
    rho = rho if rho is not None else torch.empty((b.rows,), dtype=torch.float32, device=a.device)
    need = workspace_bytes(OP_SPLIT_QUANT, rows, cols, 0, nseg)
    ws = ws if ws is not None else _workspace(need, a.device)
    r, m, cb = res.c(), mean.c(), b.c()
    _check("averis_split_quant_grouped_rank1", lib().averis_split_quant_grouped_rank1(
        a.data_ptr(), _dtype_code(a), rows, cols, _lda(a), offsets.data_ptr(), nseg, seed, rnd,
        ctypes.byref(r), ctypes.byref(m), mu.data_ptr(), ctypes.byref(cb), rho.data_ptr(),
        ws.data_ptr(), ws.numel(), _stream()))
    return res, mean, mu, rho


def averis_gemm_grouped_rank1(a, rho, b, offsets, out_dtype=torch.float32, out=None):
    """c[rows of s] = deq(a_s) deq(b_s)^T + 1 rho_s^T."""
    nseg = offsets.numel() - 1
    c = _out(a.rows, b.rows // nseg, out_dtype, a.codes.device, out)
    ca, cb = a.c(), b.c()
    _check("averis_gemm_grouped_rank1", lib().averis_gemm_grouped_rank1(
        ctypes.byref(ca), rho.data_ptr(), ctypes.byref(cb), offsets.data_ptr(), nseg,
        c.data_ptr(), _dtype_code(c), c.stride(0), _stream()))
    return c


def averis_gemm_rank1_stats(a, rho, b, ws=None, out=None):
    """averis_gemm_rank1 with bf16 output that also writes the column
    statistics of the output into ws, the split workspace of that output;
    returns (c, ws) for averis_split_quant_from_stats."""
    m, n = a.rows, b.rows
    c = _out(m, n, torch.bfloat16, a.codes.device, out)
    need = workspace_bytes(OP_SPLIT_QUANT, m, n)
    ws = ws if ws is not None else _workspace(need, a.codes.device)
    ca, cb = a.c(), b.c()
    _check("averis_gemm_rank1_stats", lib().averis_gemm_rank1_stats(
        ctypes.byref(ca), rho.data_ptr(), ctypes.byref(cb), c.data_ptr(), c.stride(0),
        ws.data_ptr(), ws.numel(), _stream()))
    return c, ws


def averis_split_quant_from_stats(c, ws, seed=0, rnd=SR, b=None, rho=None):
    """averis_split_quant of the bf16 output c of averis_gemm_rank1_stats from
    the statistics it left in ws; with b, also the rank-one row for the GEMM
    that takes this split.  Returns (residual, mean, mu_f32) or, with b,
    (residual, mean, mu_f32, rho)."""
    rows, cols = c.shape
    res = NVFP4.empty(rows, cols, 1, c.device)
    mean = NVFP4.empty(1, cols, 1, c.device)
    mu = torch.empty((cols,), dtype=torch.float32, device=c.device)
    if b is not None and rho is None:
        rho = torch.empty((b.rows,), dtype=torch.float32, device=c.device)
    r, m = res.c(), mean.c()
    cb = b.c() if b is not None else None
    _check("averis_split_quant_from_stats", lib().averis_split_quant_from_stats(
        c.data_ptr(), rows, cols, _lda(c), seed, rnd, ctypes.byref(r), ctypes.byref(m),
        mu.data_ptr(), ctypes.byref(cb) if cb is not None else None,
        rho.data_ptr() if rho is not None else None, ws.data_ptr(), ws.numel(), _stream()))
    return (res, mean, mu) if b is None else (res, mean, mu, rho)
