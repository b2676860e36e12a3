"""The Averis split-quant and quantized GEMMs, step by step (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

All inputs are float32 numpy arrays (a bf16 tensor is widened exactly to
float32 before it reaches the oracle).  Every FP32 intermediate that decides a
code or a scale byte is rounded exactly as written below (numpy float32
arithmetic is IEEE round-to-nearest-even, one rounding per operation).

Readings of the pages taken here (the pages give the equations, not the
arithmetic):

* mean ([Lighthouse] §2.1): mu_j = (1/l) sum_i a_ij over the l rows (tokens)
  of the GEMM's left operand.  Computed as float32(RN64(S_j) / l), where
  RN64(S_j) is the exact column sum correctly rounded to float64 (math.fsum)
  and the division is one float64 operation.
* residual ([Lighthouse] §2.2 and [Gist] §2): r_ij = float32(a_ij - mu_j),
  using the unquantized mean; it is quantized on its own.
* Q4 ([Lighthouse] §1.1 and §3.1; [NVFP4-outliers]): blocks of 16 along the
  GEMM contraction axis; a float32 tensor scale and an E4M3 scale per block:
    amax   = max |T| over the tensor
    S_enc  = float32(2688 / amax)  (2688 = 6 * 448), or 1 if amax == 0 or the
             quotient is not finite;  S_dec = float32(1 / S_enc)
    s_b    = float32(float32(amax_b / 6) * S_enc), capped at 448
    c_b    = E4M3(s_b) (RNE), d_b its value
    e_b    = float32(S_enc / d_b) if d_b > 0 else 0
    v_k    = float32(T_k * e_b) -> E2M1 code by RN or SR
  and the dequantized value is E2M1(code) * d_b * S_dec (exact in float64).
* SR draws come from oracle.philox keyed by (seed, stream, row * cols + col);
  streams: 0 residual / vanilla activations, 1 mean, 2 weights, 3 the
  transposed residuals of the wgrad product.
* GEMMs ([Lighthouse] §2.2): Y = 1 (deq(mean_q) deq(B)^T) + deq(X_R,q) deq(B)^T
  with B = W^T quantized along m (forward), and the same with D and B = W
  quantized along n (dgrad); the vanilla arm is deq(Q4(X)) deq(B)^T.  All
  products and sums are float64.
* wgrad (not among the pages' equations; reading): the same split applied to
  both operands of dW = X^T D.  With X = X_R + 1 mu^T and D = D_R + 1 nu^T,
  X^T D = X_R^T D_R + X_R^T 1 nu^T + mu 1^T D_R + l mu nu^T, and the two
  middle terms vanish because the residuals have zero column sums.  So
    dW = deq(Q4(X_R^T)) deq(Q4(D_R^T))^T + l mu_X nu_D^T,
  with the transposed residuals quantized in blocks of 16 along the token axis
  (the contraction axis of this product), SR stream 3, and the outer product
  taken from the fp32 means the splits already hold.  The outer product is no
  contraction, so no FP4 GEMM needs its operands quantized; quantizing them
  (mean="q4", for comparison) gives one error per column that the factor l
  multiplies coherently instead of averaging it over the tokens.
* mean-energy ratio ([Lighthouse] §7 recommends monitoring R = ||mu||_2 /
  sqrt(E||X||^2 / N) and leaves E and N open): E||X||^2 is read as the sum of
  squares of the whole operand, ||A||_F^2, and N as its row count l, so the
  denominator is the mean squared row norm and 0 <= R <= 1, with R = 1 exactly
  when every row equals mu.  Computed in float64 from exact sums (fsum); R = 0
  when l = 0 or A = 0; per segment when grouped.
* shared 16x16-block weight (the next step [Lighthouse] §2.2 suggests by
  writing the dgrad operand as the transpose of the forward one; reading):
  one quantization of W (m x n) in 16 x 16 tiles, each with one E4M3 scale
  from the tile's largest magnitude (s_b, c_b, e_b as in Q4; tensor scale from
  max |W|; SR index i * n + j, stream 2).  Both GEMM copies hold these same
  codes: the dgrad operand (m x n, blocks of 16 along n) and its transpose,
  the forward operand (n x m, blocks of 16 along m), each 16-run carrying its
  tile's scale byte, so deq(forward) = deq(dgrad)^T exactly.
* grouped (one mean and one tensor scale per expert segment): every step above
  is applied to each segment's rows; SR indices use the global row, the mean
  of segment s uses index s * cols + col; an empty segment has mean 0.
"""

import math

import numpy as np

from . import formats
from .philox import sr_draw16

BLOCK = 16
F32 = np.float32


# --------------------------------------------------------------------------
# mean and residual
# --------------------------------------------------------------------------

def column_mean(a):
    """mu_j = float32(fsum(a[:, j]) / rows) for a float32 (rows x cols) array."""
    a = np.asarray(a, dtype=np.float32)
    rows, cols = a.shape
    if rows == 0:
        return np.zeros(cols, dtype=np.float32)
    sums = np.array([math.fsum(a[:, j].astype(np.float64)) for j in range(cols)],
                    dtype=np.float64)
    return (sums / np.float64(rows)).astype(np.float32)


def residual(a, mu):
    """r = float32(a - mu) broadcast over rows."""
    return (np.asarray(a, dtype=np.float32) - np.asarray(mu, dtype=np.float32)[None, :]).astype(np.float32)


def mean_energy_ratio(a):
    """R = ||mu||_2 / sqrt(||A||_F^2 / l) for a float32 (l x m) array, float64,
    with mu the exact column mean (fsum / l); 0 for l = 0 or A = 0."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    l = a.shape[0]
    if l == 0:
        return 0.0
    mu = np.array([math.fsum(a[:, j]) / l for j in range(a.shape[1])], dtype=np.float64)
    ssq = math.fsum((a * a).ravel())    # each square is exact in float64
    if ssq == 0.0:
        return 0.0
    return math.sqrt(math.fsum(mu * mu) / (ssq / l))


# --------------------------------------------------------------------------
# Q4: NVFP4-style two-level quantization
# --------------------------------------------------------------------------

def tensor_scales(amax):
    """(S_enc, S_dec) as float32 from the tensor's float32 max magnitude."""
    amax = F32(amax)
    if amax == 0:
        s_enc = F32(1.0)
    else:
        with np.errstate(over="ignore", divide="ignore"):
            s_enc = F32(2688.0) / amax
        if not np.isfinite(s_enc):
            s_enc = F32(1.0)
    s_dec = F32(1.0) / s_enc
    return F32(s_enc), F32(s_dec)


def quantize(t, rnd="sr", seed=0, stream=0, row0=0, amax=None):
    """Q4 of a float32 (rows x cols) tensor; blocks of 16 along cols.

    row0 offsets the row used in the SR index (global row of a segment).
    amax, if given, overrides the tensor's own max magnitude (never used by the
    method itself; kept for tests of the scale arithmetic).
    Returns dict(codes=u8[rows, cols/2], scales=u8[rows, cols/16],
    s_enc=f32, s_dec=f32).
    """
    t = np.asarray(t, dtype=np.float32)
    rows, cols = t.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 16")
    if amax is None:
        amax = np.max(np.abs(t)) if t.size else F32(0.0)
    s_enc, s_dec = tensor_scales(amax)
    nb = cols // BLOCK
    blk = t.reshape(rows, nb, BLOCK)
    amax_b = np.max(np.abs(blk), axis=-1) if rows else np.zeros((0, nb), np.float32)
    s_b = ((amax_b / F32(6.0)).astype(np.float32) * s_enc).astype(np.float32)
    s_b = np.minimum(s_b, F32(formats.E4M3_MAX))
    c_b = formats.e4m3_encode(s_b)
    d_b = formats.e4m3_decode(c_b).astype(np.float32)       # exact in float32
    with np.errstate(divide="ignore"):
        e_b = np.where(d_b > 0, s_enc / np.where(d_b > 0, d_b, F32(1.0)), F32(0.0)).astype(np.float32)
    v = (blk * e_b[..., None]).astype(np.float32).reshape(rows, cols)
    if rnd == "rn":
        codes = formats.e2m1_round_rn(v)
    elif rnd == "sr":
        r_idx = (np.arange(rows, dtype=np.uint64) + np.uint64(row0))[:, None]
        idx = r_idx * np.uint64(cols) + np.arange(cols, dtype=np.uint64)[None, :]
        codes = formats.e2m1_round_sr(v, sr_draw16(seed, stream, idx))
    else:
        raise ValueError("rnd must be 'rn' or 'sr'")
    return dict(codes=formats.pack_nibbles(codes), scales=c_b, s_enc=s_enc, s_dec=s_dec)


def dequantize(q):
    """float64 values of an oracle-quantized tensor (exact)."""
    codes = formats.unpack_nibbles(q["codes"])
    rows, cols = codes.shape
    d = formats.e4m3_decode(q["scales"]).astype(np.float64)
    vals = formats.e2m1_decode(codes).reshape(rows, cols // BLOCK, BLOCK) * d[..., None]
    return vals.reshape(rows, cols) * np.float64(q["s_dec"])


# --------------------------------------------------------------------------
# Averis split-quant, vanilla quant, weight quant
# --------------------------------------------------------------------------

def split_quant(a, rnd="sr", seed=0):
    """mu, X_R,q = Q4(a - 1 mu) (stream 0), mean_q = Q4(mu) (stream 1)."""
    a = np.asarray(a, dtype=np.float32)
    mu = column_mean(a)
    r = residual(a, mu)
    res_q = quantize(r, rnd, seed, stream=0)
    mean_q = quantize(mu[None, :], rnd, seed, stream=1)
    return dict(mu=mu, residual=res_q, mean=mean_q)


def vanilla_quant(a, rnd="sr", seed=0):
    """Q4 of the activation itself, no split (stream 0)."""
    return quantize(np.asarray(a, dtype=np.float32), rnd, seed, stream=0)


def weight_quant(w, rnd="rn", seed=0):
    """The two quantized copies of W (m x n): forward B = Q4(W^T) (n x m, blocks
    along m) and dgrad B = Q4(W) (m x n, blocks along n); stream 2."""
    w = np.asarray(w, dtype=np.float32)
    return dict(fwd=quantize(np.ascontiguousarray(w.T), rnd, seed, stream=2),
                dgrad=quantize(w, rnd, seed, stream=2))


def weight_quant_2d(w, rnd="rn", seed=0, stream=2, row0=0):
    """The shared 16x16-block quantization of W (m x n): returns dict(fwd=...,
    dgrad=...) in the format of quantize(), fwd = n x m (the transpose) and
    dgrad = m x n, with the same codes and one scale per 16 x 16 tile.  row0
    offsets the row in the SR index (matrix b of a batch: b * m)."""
    w = np.asarray(w, dtype=np.float32)
    m, n = w.shape
    if m % BLOCK or n % BLOCK:
        raise ValueError("rows and cols must be multiples of 16")
    amax = np.max(np.abs(w)) if w.size else F32(0.0)
    s_enc, s_dec = tensor_scales(amax)
    tiles = w.reshape(m // BLOCK, BLOCK, n // BLOCK, BLOCK)
    amax_t = np.max(np.abs(tiles), axis=(1, 3))                       # (m/16, n/16)
    s_t = ((amax_t / F32(6.0)).astype(np.float32) * s_enc).astype(np.float32)
    s_t = np.minimum(s_t, F32(formats.E4M3_MAX))
    c_t = formats.e4m3_encode(s_t)
    d_t = formats.e4m3_decode(c_t).astype(np.float32)
    with np.errstate(divide="ignore"):
        e_t = np.where(d_t > 0, s_enc / np.where(d_t > 0, d_t, F32(1.0)), F32(0.0)).astype(np.float32)
    v = (tiles * e_t[:, None, :, None]).astype(np.float32).reshape(m, n)
    if rnd == "rn":
        codes = formats.e2m1_round_rn(v)
    elif rnd == "sr":
        r_idx = (np.arange(m, dtype=np.uint64) + np.uint64(row0))[:, None]
        idx = r_idx * np.uint64(n) + np.arange(n, dtype=np.uint64)[None, :]
        codes = formats.e2m1_round_sr(v, sr_draw16(seed, stream, idx))
    else:
        raise ValueError("rnd must be 'rn' or 'sr'")
    dgrad = dict(codes=formats.pack_nibbles(codes), scales=np.repeat(c_t, BLOCK, axis=0),
                 s_enc=s_enc, s_dec=s_dec)
    fwd = dict(codes=formats.pack_nibbles(np.ascontiguousarray(codes.T)),
               scales=np.repeat(np.ascontiguousarray(c_t.T), BLOCK, axis=0), s_enc=s_enc, s_dec=s_dec)
    return dict(fwd=fwd, dgrad=dgrad)


# --------------------------------------------------------------------------
# GEMMs (float64)
# --------------------------------------------------------------------------

def gemm(a_q, b_q, mean_q=None):
    """deq(A) deq(B)^T (+ 1 (deq(mean) deq(B)^T) if a quantized mean is given)."""
    b = dequantize(b_q)
    c = dequantize(a_q) @ b.T
    if mean_q is not None:
        c = c + (dequantize(mean_q) @ b.T)[0][None, :]
    return c


def gemm_abs_bound(a_q, b_q, mean_q=None):
    """|deq A| |deq B|^T (+ |deq mean| |deq B|^T): the scale the GEMM error is
    measured against (an FP32-accumulated result is within K * 2^-24 of it)."""
    b = np.abs(dequantize(b_q))
    c = np.abs(dequantize(a_q)) @ b.T
    if mean_q is not None:
        c = c + (np.abs(dequantize(mean_q)) @ b.T)[0][None, :]
    return c


def averis_forward(x, w_q_fwd, rnd="sr", seed=0):
    """Y = 1 (mean_q W_q) + X_R,q W_q ([Lighthouse] §2.2, forward)."""
    s = split_quant(x, rnd, seed)
    return s, gemm(s["residual"], w_q_fwd, s["mean"])


def averis_dgrad(d, w_q_dgrad, rnd="sr", seed=0):
    """dX = 1 (mean_q,D W_q^T) + D_R,q W_q^T ([Lighthouse] §2.2, backward)."""
    s = split_quant(d, rnd, seed)
    return s, gemm(s["residual"], w_q_dgrad, s["mean"])


def vanilla_forward(x, w_q_fwd, rnd="sr", seed=0):
    """Comparison arm ([Abstract]: vanilla NVFP4): deq(Q4(X)) deq(W_q)."""
    q = vanilla_quant(x, rnd, seed)
    return q, gemm(q, w_q_fwd)


# --------------------------------------------------------------------------
# wgrad (reading: the split applied to both operands of X^T D)
# --------------------------------------------------------------------------

def residual_t_quant(a, mu, rnd="sr", seed=0):
    """Q4 of the transposed residual (cols x rows, blocks of 16 along the rows,
    i.e. the token axis), SR stream 3: the wgrad operand."""
    r = residual(np.asarray(a, dtype=np.float32), mu)
    return quantize(np.ascontiguousarray(r.T), rnd, seed, stream=3)


def wgrad_combine(xt, dt, mean_x, mean_d, l):
    """xt dt^T + l mean_x^T mean_d for float64 operands: xt (m x l), dt (n x l),
    mean_x (m,), mean_d (n,).  The quantized wgrad feeds it dequantized values;
    with exact residuals and means it reproduces X^T D."""
    return xt @ dt.T + np.float64(l) * np.outer(mean_x, mean_d)


def averis_wgrad(x, d, rnd="sr", seed_x=0, seed_d=0, mean="f32"):
    """dW (m x n) for X (l x m) and D (l x n): the splits of X and D (seeds as
    in the forward and dgrad passes), the transposed residuals quantized along
    the tokens, and the outer product of the fp32 means (mean="f32") or of the
    dequantized FP4 means (mean="q4")."""
    x = np.asarray(x, dtype=np.float32)
    d = np.asarray(d, dtype=np.float32)
    sx, sd = split_quant(x, rnd, seed_x), split_quant(d, rnd, seed_d)
    xt = residual_t_quant(x, sx["mu"], rnd, seed_x)
    dt = residual_t_quant(d, sd["mu"], rnd, seed_d)
    if mean == "f32":
        mx, md = sx["mu"].astype(np.float64), sd["mu"].astype(np.float64)
    elif mean == "q4":
        mx, md = dequantize(sx["mean"])[0], dequantize(sd["mean"])[0]
    else:
        raise ValueError("mean must be 'f32' or 'q4'")
    dw = wgrad_combine(dequantize(xt), dequantize(dt), mx, md, x.shape[0])
    return dict(xt=xt, dt=dt, mu_x=sx["mu"], mu_d=sd["mu"], dw=dw)


def wgrad_abs_bound(xt, dt, mu_x, mu_d, l):
    """|deq xt| |deq dt|^T + l |mu_x| |mu_d|^T: the scale the wgrad error is
    measured against."""
    return wgrad_combine(np.abs(dequantize(xt)), np.abs(dequantize(dt)),
                         np.abs(np.asarray(mu_x, np.float64)), np.abs(np.asarray(mu_d, np.float64)), l)


# --------------------------------------------------------------------------
# grouped (expert segments)
# --------------------------------------------------------------------------

def split_quant_grouped(a, offsets, rnd="sr", seed=0):
    """Per-segment split-quant over rows offsets[s]:offsets[s+1]."""
    a = np.asarray(a, dtype=np.float32)
    rows, cols = a.shape
    nseg = len(offsets) - 1
    mu = np.zeros((nseg, cols), dtype=np.float32)
    res = []
    means = []
    for s in range(nseg):
        r0, r1 = int(offsets[s]), int(offsets[s + 1])
        seg = a[r0:r1]
        if r1 > r0:
            mu[s] = column_mean(seg)
        res.append(quantize(residual(seg, mu[s]), rnd, seed, stream=0, row0=r0))
        m = quantize(mu[s][None, :], rnd, seed, stream=1, row0=s)
        means.append(m)
    return dict(mu=mu, residual=res, mean=means)


def mean_energy_ratio_grouped(a, offsets):
    """R of each segment's rows (0 for an empty segment)."""
    a = np.asarray(a, dtype=np.float32)
    return np.array([mean_energy_ratio(a[int(offsets[s]):int(offsets[s + 1])])
                     for s in range(len(offsets) - 1)], dtype=np.float64)


def vanilla_quant_grouped(a, offsets, rnd="sr", seed=0):
    a = np.asarray(a, dtype=np.float32)
    return [quantize(a[int(offsets[s]):int(offsets[s + 1])], rnd, seed, stream=0, row0=int(offsets[s]))
            for s in range(len(offsets) - 1)]


def gemm_grouped(a_qs, b_qs, mean_qs=None):
    """Row-concatenation over segments of gemm(a_q[s], b_q[s], mean_q[s])."""
    outs = []
    for s in range(len(a_qs)):
        outs.append(gemm(a_qs[s], b_qs[s], None if mean_qs is None else mean_qs[s]))
    return np.concatenate(outs, axis=0)
