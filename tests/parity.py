"""Shared parity criteria of the GPU tests, and a process pool that runs the
oracle's quantization over row blocks of a large tensor in parallel.

GEMM acceptance: a relative error of at most 1e-3 against the oracle's
float64 product of the same dequantized operands, read two ways, both
required for fp32 output:
  * elementwise: |C - C_ref| <= 1e-3 (|deq A| |deq B|^T + 1 |deq mean| |deq B|^T),
    the scale on which an FP32-accumulated product of exact operands is measured
    where C_ref cancels to ~0;
  * normwise: max |C - C_ref| <= 1e-3 max |C_ref|.
bf16 output adds its own rounding (half an ulp, at most 2^-9 relative) to the
elementwise test and is not held to the normwise one.

The pool only splits work: every block is one call of oracle.averis.quantize
with the tensor's own amax and the block's first global row (row0), which is
exactly how a whole-tensor call treats those rows (the SR index depends only
on the global element index, pinned in tests/test_oracle_quant.py)."""

import multiprocessing as mp
import os

import numpy as np

GEMM_TOL = 1e-3
BF16_REL = 2.0 ** -8


def assert_quant_equal(gpu, ref, seg=0, rows=None):
    """Codes, scale bytes and the tensor scale of segment `seg` bit-exact."""
    g = gpu.cpu() if hasattr(gpu, "cpu") else gpu
    codes, scales = g["codes"], g["scales"]
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    np.testing.assert_array_equal(codes, ref["codes"])
    np.testing.assert_array_equal(scales, ref["scales"])
    assert g["tscale"][2 * seg] == ref["s_enc"]
    assert g["tscale"][2 * seg + 1] == ref["s_dec"]


def gemm_errors(c, ref, bound):
    """(max elementwise error / bound, max |C - C_ref| / max |C_ref|)."""
    err = np.abs(np.asarray(c, dtype=np.float64) - ref)
    elem = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    peak = float(np.max(np.abs(ref))) if ref.size else 0.0
    norm = float(np.max(err)) / peak if peak > 0 else float(np.max(err, initial=0.0))
    return elem, norm


def assert_elementwise(c, ref, bound, bf16=False):
    c = np.asarray(c, dtype=np.float64)
    lim = GEMM_TOL * bound + (BF16_REL * np.abs(ref) if bf16 else 0.0)
    ok = np.abs(c - ref) <= lim
    assert ok.all(), "max |C - ref| / bound = %.3g" % gemm_errors(c, ref, bound)[0]


def assert_normwise(c, ref):
    c = np.asarray(c, dtype=np.float64)
    peak = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(c - ref))) if ref.size else 0.0
    assert err <= GEMM_TOL * peak, "max |C - ref| / max |ref| = %.3g" % (err / max(peak, 1e-300))


def assert_gemm_close(c, ref, bound, bf16=False, label=""):
    """The acceptance test above; c: numpy array or torch tensor."""
    if hasattr(c, "float"):
        c = c.float().cpu().numpy()
    c = np.asarray(c, dtype=np.float64)
    if label:
        elem, norm = gemm_errors(c, ref, bound)
        print("%s: max err/bound %.3g, max err/max|ref| %.3g" % (label, elem, norm), flush=True)
    assert_elementwise(c, ref, bound, bf16)
    if not bf16:
        assert_normwise(c, ref)


# --------------------------------------------------------------------------
# the oracle over row blocks, in worker processes
# --------------------------------------------------------------------------

def _quantize_block(args):
    from oracle import averis as orc
    r, rnd, seed, stream, row0, amax = args
    return orc.quantize(r, rnd, seed, stream=stream, row0=row0, amax=amax)


class OraclePool:
    """Spawned worker processes (numpy only; they never touch the GPU)."""

    def __init__(self, procs=None):
        n = procs or min(16, len(os.sched_getaffinity(0)))
        self.pool = mp.get_context("spawn").Pool(max(1, n))

    def close(self):
        self.pool.terminate()
        self.pool.join()

    def quantize(self, r, rnd, seed, stream, row0=0, amax=None, block=512):
        """oracle.quantize(r, rnd, seed, stream, row0, amax) computed over
        blocks of `block` rows; amax defaults to max |r| (the tensor's own)."""
        return self.quantize_many([(r, rnd, seed, stream, row0, amax)], block)[0]

    def quantize_many(self, calls, block=512):
        """Several such calls, (r, rnd, seed, stream, row0, amax) each, with
        all their blocks in one map."""
        jobs, spans = [], []
        for r, rnd, seed, stream, row0, amax in calls:
            r = np.ascontiguousarray(r, dtype=np.float32)
            if amax is None:
                amax = np.max(np.abs(r)) if r.size else np.float32(0.0)
            first = len(jobs)
            jobs += [(r[b:b + block], rnd, seed, stream, row0 + b, amax)
                     for b in range(0, max(r.shape[0], 1), block)]
            spans.append((first, len(jobs)))
        parts = self.pool.map(_quantize_block, jobs, chunksize=1)
        out = []
        for a, b in spans:
            ps = parts[a:b]
            out.append(dict(codes=np.concatenate([p["codes"] for p in ps]),
                            scales=np.concatenate([p["scales"] for p in ps]),
                            s_enc=ps[0]["s_enc"], s_dec=ps[0]["s_dec"]))
        return out
