"""C-ABI checks that need no GPU: the library loads, exports every function
include/averis.h declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from mean_residual_quantized_amd import averis as av

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# stand-in device addresses: validation must reject the call before using them
P = 0x10000
P2 = 0x20000


def header_functions():
    src = open(os.path.join(ROOT, "include", "averis.h")).read()
    return sorted(set(re.findall(r"\b(averis_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return av.lib()


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert sorted(av.EXPORTS) == names


def test_version_and_status_strings(L):
    assert L.averis_abi_version() == 1
    for s in range(8):
        assert L.averis_status_str(s)
    assert b"unknown" in L.averis_status_str(99)


def test_workspace_queries(L):
    wb = av.workspace_bytes
    assert wb(av.OP_SPLIT_QUANT, 8192, 1024) > 0
    assert wb(av.OP_SPLIT_QUANT, 8192, 24) == 0          # cols % 16
    assert wb(av.OP_SPLIT_QUANT, -1, 32) == 0
    assert wb(av.OP_GEMM, 8192, 1024, 3072) >= 3072 * 4
    assert wb(av.OP_GEMM, 8192, 1024, 3072, 64) >= 64 * 3072 * 4
    assert wb(av.OP_QUANT, 64, 128, 0, 8) > 0
    assert wb(av.OP_QUANT_PAIR_MULTI, 0, 0, 7) == 7 * 1024 * 4
    assert wb(av.OP_QUANT_PAIR_MULTI, 0, 0, 0) == 0
    assert wb(av.OP_QUANT_PAIR_MULTI, 0, 0, av.MAX_WEIGHTS + 1) == 0
    # grows with the grouped segment count
    assert wb(av.OP_SPLIT_QUANT, 4096, 256, 0, 64) > wb(av.OP_SPLIT_QUANT, 4096, 256, 0, 1)


def nv(rows, cols, codes=P, scales=P2, tscale=P):
    return av._NVFP4(codes, scales, tscale, rows, cols)


def split(L, a=P, dtype=av.BF16, rows=64, cols=128, lda=128, rnd=av.SR, res=None, mean=None,
          mu=None, ws=P, wsb=1 << 30):
    res = res if res is not None else nv(rows, cols)
    mean = mean if mean is not None else nv(1, cols)
    return L.averis_split_quant(a, dtype, rows, cols, lda, 0, rnd, ctypes.byref(res),
                                ctypes.byref(mean), mu, ws, wsb, None)


def test_split_quant_rejections(L):
    assert split(L, cols=24, lda=24) == 2                 # cols % 16
    assert split(L, cols=0, lda=0) == 2
    assert split(L, rows=-1) == 2
    assert split(L, lda=64) == 2                          # lda < cols
    assert split(L, dtype=7) == 3
    assert split(L, a=None) == 1
    assert split(L, a=P + 2) == 4                         # misaligned input
    assert split(L, lda=132) == 4                         # row stride not 16-byte multiple
    assert split(L, rnd=5) == 6
    assert split(L, res=nv(64, 64)) == 2                  # residual shape mismatch
    assert split(L, mean=nv(2, 128)) == 2
    assert split(L, res=nv(64, 128, codes=None)) == 1
    assert split(L, res=nv(64, 128, codes=P + 8)) == 4
    assert split(L, ws=None) == 5
    assert split(L, wsb=16) == 5
    assert split(L, ws=P + 16) == 4                       # workspace alignment


def test_split_rank1_multi_rejections(L):
    res, mean = nv(64, 128), nv(1, 128)

    def rm(nb=2, bs=None, rhos=None, cols=128, lda=128, **kw):
        bs = bs if bs is not None else [nv(96, cols), nv(32, cols)]
        rhos = rhos if rhos is not None else [P, P2]
        barr = (ctypes.POINTER(av._NVFP4) * len(bs))(
            *[ctypes.pointer(b) if b is not None else None for b in bs])
        rarr = (ctypes.c_void_p * len(rhos))(*rhos)
        return L.averis_split_quant_rank1_multi(
            kw.get("a", P), av.BF16, 64, cols, lda, 0, av.SR, ctypes.byref(res),
            ctypes.byref(mean), P, nb, ctypes.cast(barr, ctypes.c_void_p),
            ctypes.cast(rarr, ctypes.c_void_p), kw.get("ws", P), 1 << 30, None)
    nul = ctypes.c_void_p(None)
    assert L.averis_split_quant_rank1_multi(P, av.BF16, 64, 128, 128, 0, av.SR, ctypes.byref(res),
                                            ctypes.byref(mean), P, 2, None, P, P, 1 << 30,
                                            None) == 1
    assert rm(nb=0) == 6
    assert rm(nb=5, bs=[nv(16, 128)] * 5, rhos=[P] * 5) == 6   # AVERIS_MAX_RANK1
    assert rm(bs=[nv(96, 128), None]) == 1                    # every entry checked
    assert rm(rhos=[P, 0]) == 1
    assert rm(rhos=[P, P + 2]) == 4                           # 4-byte rho
    assert rm(bs=[nv(96, 128), nv(32, 64)]) == 2              # b[i]->cols == cols
    assert rm(bs=[nv(96, 128), nv(0, 128)]) == 2              # an empty b
    assert rm(bs=[nv(96, 128), nv(32, 128, codes=P + 8)]) == 4
    assert rm(a=P + 2) == 4                                   # then the split's own checks
    assert rm(ws=None) == 5
    del nul


def test_noalloc_split_rejections(L):
    # the argument checks of averis_split_quant, and inputs whose
    # intermediate results do not fit the library's device array, all before
    # any HIP call (this host has no GPU)
    sq = lambda a=P, dtype=av.BF16, rows=64, cols=128, lda=128, rnd=av.SR, res=None, mean=None: \
        L.averis_split_quant_noalloc(a, dtype, rows, cols, lda, 0, rnd,
                                     ctypes.byref(res if res is not None else nv(rows, cols)),
                                     ctypes.byref(mean if mean is not None else nv(1, cols)),
                                     None, None)
    assert sq(cols=24, lda=24) == 2
    assert sq(dtype=7) == 3
    assert sq(a=None) == 1
    assert sq(a=P + 2) == 4
    assert sq(rnd=5) == 6
    assert sq(res=nv(64, 64)) == 2
    limit = 16 << 20
    rows, cols = 32768, 3072
    assert av.workspace_bytes(av.OP_SPLIT_QUANT, rows, cols) > limit
    assert sq(rows=rows, cols=cols, lda=cols) == 5
    msg = L.averis_last_error().decode()
    assert "noalloc" in msg and str(limit) in msg, msg
    assert av.workspace_bytes(av.OP_SPLIT_QUANT, 16384, 3072) <= limit


def test_fused_statistics_rejections(L):
    a, b = nv(1000, 128), nv(208, 128)
    g = lambda a=a, rho=P, b=b, c=P, ldc=208, ws=P, wsb=1 << 30: L.averis_gemm_rank1_stats(
        ctypes.byref(a) if a is not None else None, rho, ctypes.byref(b), c, ldc, ws, wsb, None)
    assert g(a=None) == 1
    assert g(rho=None) == 1
    assert g(a=nv(1000, 96), b=nv(208, 96)) == 2          # K % 64 (the fused epilogue's kernel)
    assert g(b=nv(200, 128)) == 2                          # output cols % 16 (a split input)
    assert g(ldc=100) == 2
    assert g(c=None) == 1
    assert g(c=P + 4) == 4                                 # a split input is 16-byte aligned
    assert g(ldc=212) == 4                                 # ... with 16-byte rows
    assert g(ws=None) == 5
    assert g(wsb=64) == 5
    res, mean = nv(1000, 208), nv(1, 208)
    sq = lambda a=P, rows=1000, cols=208, lda=208, rnd=av.SR, res=res, b=None, rho=None, ws=P, \
        wsb=1 << 30: L.averis_split_quant_from_stats(
            a, rows, cols, lda, 0, rnd, ctypes.byref(res), ctypes.byref(mean), None,
            ctypes.byref(b) if b is not None else None, rho, ws, wsb, None)
    assert sq(cols=200, lda=200) == 2
    assert sq(a=None) == 1
    assert sq(rnd=4) == 6
    assert sq(res=nv(999, 208)) == 2
    assert sq(b=nv(96, 208)) == 1                          # b without rho
    assert sq(rho=P) == 1                                  # rho without b
    assert sq(b=nv(96, 200), rho=P) == 2
    assert sq(ws=None) == 5


def test_quant_and_gemm_rejections(L):
    out = nv(64, 128)
    q = lambda **k: L.averis_quant(k.get("a", P), k.get("dt", av.BF16), k.get("rows", 64),
                                   k.get("cols", 128), k.get("lda", 128), k.get("tr", 0), 0,
                                   k.get("rnd", av.SR), k.get("stream", 0),
                                   ctypes.byref(k.get("out", out)), P, 1 << 30, None)
    assert q(cols=40, lda=40) == 2
    assert q(tr=2) == 6
    assert q(stream=1 << 20) == 6
    assert q(tr=1, lda=32) == 2                           # transposed: lda >= rows
    assert q(out=nv(64, 64)) == 2
    assert q(dt=9) == 3

    a, b, m = nv(64, 128), nv(32, 128), nv(1, 128)
    g = lambda a=a, m=m, b=b, c=P, dt=av.F32, ldc=32, ws=P, wsb=1 << 20: L.averis_gemm_fwd(
        ctypes.byref(a), None if m is None else ctypes.byref(m), ctypes.byref(b), c, dt, ldc, ws,
        wsb, None)
    assert g(b=nv(32, 64)) == 2                           # K mismatch
    assert g(m=None) == 1
    assert g(m=nv(1, 64)) == 2
    assert g(ldc=16) == 2
    assert g(c=None) == 1
    assert g(dt=4) == 3
    assert g(ws=None) == 5
    assert g(wsb=8) == 5
    assert g(a=nv(64, 120)) == 2                          # K % 16
    assert L.averis_gemm_vanilla(ctypes.byref(a), ctypes.byref(b), P + 2, av.F32, 32, None, 0,
                                 None) == 4
    # grouped: B rows must be a multiple of nseg, offsets required
    assert L.averis_gemm_grouped(ctypes.byref(a), None, ctypes.byref(nv(33, 128)), P, 2, P,
                                 av.F32, 32, P, 1 << 20, None) == 2
    assert L.averis_gemm_grouped(ctypes.byref(a), None, ctypes.byref(b), None, 2, P, av.F32, 32,
                                 P, 1 << 20, None) == 1
    assert L.averis_gemm_grouped(ctypes.byref(a), None, ctypes.byref(b), P, 0, P, av.F32, 32, P,
                                 1 << 20, None) == 6


def test_grouped_and_batched_rejections(L):
    res, mean = nv(64, 128), nv(4, 128)
    sg = lambda offs=P, nseg=4, mean=mean: L.averis_split_quant_grouped(
        P, av.BF16, 64, 128, 128, offs, nseg, 0, av.SR, ctypes.byref(res), ctypes.byref(mean),
        None, P, 1 << 30, None)
    assert sg(offs=None) == 1
    assert sg(offs=P + 4) == 4
    assert sg(nseg=0) == 6
    assert sg(nseg=5000) == 6
    assert sg(mean=nv(3, 128)) == 2
    out = nv(2 * 64, 128)
    qb = lambda batch=2, bstride=64 * 128, tr=0: L.averis_quant_batched(
        P, av.BF16, batch, 64, 128, 128, bstride, tr, 0, av.RN, 2, ctypes.byref(out), P, 1 << 20,
        None)
    assert qb(batch=0) == 6
    assert qb(bstride=100) == 2                           # overlapping batch entries
    assert qb(batch=3) == 2                               # out rows != batch * rows


def test_quant_pair_rejections(L):
    out, out_t = nv(2 * 64, 128), nv(2 * 128, 64)
    qp = lambda a=P, dt=av.BF16, batch=2, rows=64, cols=128, lda=128, bstride=64 * 128, rnd=av.RN, \
        out=out, out_t=out_t, ws=P, wsb=1 << 20: L.averis_quant_pair(
            a, dt, batch, rows, cols, lda, bstride, 0, rnd, 2, ctypes.byref(out),
            ctypes.byref(out_t), ws, wsb, None)
    assert qp(batch=0) == 6
    assert qp(rnd=3) == 6
    assert qp(dt=5) == 3
    assert qp(rows=40) == 2                               # rows % 16 (out_t's block dim)
    assert qp(cols=24, lda=24) == 2
    assert qp(lda=64) == 2
    assert qp(bstride=100) == 2                           # overlapping batch entries
    assert qp(a=None) == 1
    assert qp(a=P + 4) == 4                               # 16-byte vector loads
    assert qp(lda=132, bstride=64 * 132) == 4
    assert qp(out_t=nv(2 * 128, 32)) == 2                 # out_t is (batch*cols) x rows
    assert qp(out=nv(64, 128)) == 2
    assert qp(ws=None) == 5
    assert qp(wsb=64) == 5


def test_quant_pair_2d_rejections(L):
    out, out_t = nv(2 * 64, 128), nv(2 * 128, 64)
    qp = lambda a=P, dt=av.BF16, batch=2, rows=64, cols=128, lda=128, bstride=64 * 128, rnd=av.RN, \
        out=out, out_t=out_t, ws=P, wsb=1 << 20: L.averis_quant_pair_2d(
            a, dt, batch, rows, cols, lda, bstride, 0, rnd, 2, ctypes.byref(out),
            ctypes.byref(out_t), ws, wsb, None)
    assert qp(batch=0) == 6
    assert qp(rnd=3) == 6
    assert qp(dt=5) == 3
    assert qp(rows=40) == 2                               # 16 x 16 tiles
    assert qp(cols=24, lda=24) == 2
    assert qp(bstride=100) == 2
    assert qp(a=None) == 1
    assert qp(a=P + 4) == 4
    assert qp(out_t=nv(2 * 128, 32)) == 2
    assert qp(out=nv(64, 128)) == 2
    assert qp(ws=None) == 5
    assert qp(wsb=64) == 5


def test_quant_pair_multi_rejections(L):
    outs = [(nv(64, 128), nv(128, 64)), (nv(32, 48), nv(48, 32))]

    def qm(n=2, dt=av.BF16, rnd=av.RN, stream=2, ws=P, wsb=1 << 20, **bad):
        arr = (av._Weight * 2)()
        for i, (rows, cols) in enumerate(((64, 128), (32, 48))):
            o, ot = outs[i]
            e = dict(a=P, rows=rows, cols=cols, lda=cols, out=ctypes.pointer(o),
                     out_t=ctypes.pointer(ot))
            if i == 1:
                e.update(bad)
            arr[i] = av._Weight(e["a"], e["rows"], e["cols"], e["lda"], 0, e["out"], e["out_t"])
        return L.averis_quant_pair_multi(n, ctypes.cast(arr, ctypes.c_void_p), dt, rnd, stream,
                                         ws, wsb, None)
    assert L.averis_quant_pair_multi(2, None, av.BF16, av.RN, 2, P, 1 << 20, None) == 1
    assert qm(n=0) == 6
    assert qm(n=17) == 6                                  # AVERIS_MAX_WEIGHTS
    assert qm(dt=5) == 3
    assert qm(rnd=3) == 6
    assert qm(stream=1 << 16) == 6
    # any entry's fault rejects the whole call (the second one here)
    assert qm(rows=40) == 2                               # rows % 16
    assert qm(cols=24, lda=24) == 2
    assert qm(lda=16) == 2                                # lda < cols
    assert qm(a=None) == 1
    assert qm(a=P + 4) == 4
    assert qm(lda=52) == 4                                # 16-byte rows
    assert qm(out=ctypes.pointer(nv(32, 64))) == 2        # out is rows x cols
    assert qm(out_t=ctypes.pointer(nv(32, 48))) == 2      # out_t is cols x rows
    assert qm(out=None) == 1
    assert qm(ws=None) == 5
    assert qm(wsb=2 * 1024 * 4 - 4) == 5                  # n x 1024 floats
    assert qm(ws=P + 16) == 4


def test_wgrad_rejections(L):
    # transposed residual quant: out_t is cols x rows, rows (tokens) % 16
    out_t = nv(128, 64)
    rt = lambda a=P, dt=av.BF16, rows=64, cols=128, lda=128, mu=P, tsc=P, rnd=av.SR, out=out_t: \
        L.averis_residual_t_quant(a, dt, rows, cols, lda, mu, tsc, 0, rnd, ctypes.byref(out), None)
    assert rt(rows=40, out=nv(128, 40)) == 2
    assert rt(cols=24, lda=24) == 2
    assert rt(out=nv(64, 128)) == 2                       # not transposed
    assert rt(mu=None) == 1
    assert rt(tsc=None) == 1
    assert rt(mu=P + 4) == 4                              # 16-byte vector loads of mu
    assert rt(rnd=2) == 6
    assert rt(dt=7) == 3
    assert rt(a=None) == 1
    # wgrad GEMM: xt m x l, dt n x l, means, output m x n
    xt, dtq = nv(64, 256), nv(96, 256)
    wg = lambda xt=xt, dtq=dtq, mx=P, md=P, c=P, dt=av.F32, ld=96, ws=P, wsb=1 << 30: \
        L.averis_gemm_wgrad(ctypes.byref(xt), ctypes.byref(dtq), mx, md, c, dt, ld, ws, wsb, None)
    assert wg(dtq=nv(96, 128)) == 2                       # token counts differ
    assert wg(xt=nv(64, 200)) == 2                        # l % 16
    assert wg(dtq=nv(90, 256)) == 2                       # n % 16
    assert wg(mx=None) == 1
    assert wg(md=P + 8) == 4
    assert wg(ld=64) == 2
    assert wg(c=None) == 1
    assert wg(dt=3) == 3
    assert wg(ws=None) == 5
    assert wg(wsb=1024) == 5
    assert wg(ws=P + 64) == 4
    wb = av.workspace_bytes
    # one fp32 partial per split of the tokens; 64 tiles of 256 x 192 take 4
    assert wb(av.OP_WGRAD, 1024, 8192, 3072) == 4 * 1024 * 3072 * 4
    assert wb(av.OP_WGRAD, 64, 1008, 96) == 64 * 96 * 4  # l % 64 != 0: one partial
    assert wb(av.OP_WGRAD, 64, 0, 96) == 64 * 96 * 4


def test_split_ratio_rejections(L):
    res, mean = nv(64, 128), nv(1, 128)
    sr = lambda offs=None, nseg=1, ratio=P, mean=mean: L.averis_split_quant_ratio(
        P, av.BF16, 64, 128, 128, offs, nseg, 0, av.SR, ctypes.byref(res), ctypes.byref(mean),
        None, ratio, P, 1 << 30, None)
    assert sr(ratio=None) == 1
    assert sr(ratio=P + 2) == 4
    assert sr(nseg=2) == 6                                # no offsets: one segment
    assert sr(offs=P + 4, nseg=4, mean=nv(4, 128)) == 4
    assert sr(offs=P, nseg=4, mean=nv(3, 128)) == 2


def test_rank1_rejections(L):
    res, mean = nv(64, 128), nv(1, 128)
    b = nv(96, 128)
    sq = lambda b=b, rho=P, cols=128: L.averis_split_quant_rank1(
        P, av.BF16, 64, cols, cols, 0, av.SR, ctypes.byref(res), ctypes.byref(mean), None,
        ctypes.byref(b) if b is not None else None, rho, P, 1 << 30, None)
    assert sq(b=None) == 1
    assert sq(rho=None) == 1
    assert sq(rho=P + 2) == 4
    assert sq(b=nv(96, 64)) == 2                          # B's K differs
    assert sq(b=nv(0, 128)) == 2
    a = nv(64, 128)
    g = lambda a=a, b=b, rho=P, c=P, ldc=96, dt=av.F32: L.averis_gemm_rank1(
        ctypes.byref(a), rho, ctypes.byref(b), c, dt, ldc, None)
    assert g(rho=None) == 1
    assert g(b=nv(96, 64)) == 2
    assert g(ldc=32) == 2
    assert g(dt=2) == 3
    assert g(c=None) == 1
    assert g(rho=P + 1) == 4


def test_grouped_rank1_rejections(L):
    res, mean, b = nv(64, 128), nv(4, 128), nv(4 * 96, 128)
    sq = lambda offs=P, nseg=4, b=b: L.averis_split_quant_grouped_rank1(
        P, av.BF16, 64, 128, 128, offs, nseg, 0, av.SR, ctypes.byref(res), ctypes.byref(mean),
        None, ctypes.byref(b), P, P, 1 << 30, None)
    assert sq(offs=None) == 1
    assert sq(offs=P + 4) == 4
    assert sq(b=nv(4 * 96 + 1, 128)) == 2                 # B rows a multiple of nseg
    assert sq(nseg=0) == 6
    a = nv(64, 128)
    g = lambda offs=P, nseg=4, b=b, ldc=96: L.averis_gemm_grouped_rank1(
        ctypes.byref(a), P, ctypes.byref(b), offs, nseg, P, av.F32, ldc, None)
    assert g(offs=None) == 1
    assert g(nseg=5) == 2
    assert g(ldc=64) == 2
    assert g(nseg=0) == 6
