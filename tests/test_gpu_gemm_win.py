"""GPU parity of the GEMM whose 4-bit operands are staged in LDS as codes
(K % 256 == 0), through the C ABI: C = deq(A) deq(B)^T + 1 rho^T (rank-one
row given), deq(A) deq(B)^T (vanilla) and deq(A) deq(B)^T + 1 deq(mean)
deq(B)^T (the mean's term from its own GEMV), against the oracle's float64
product of the same bytes, to the acceptance bound of tests/parity.py.

The shapes select each of the kernel's tile widths (64 x 4, 3 and 2 output
columns: the widest tile that needs no more rounds over the 256 CUs), with
rows and columns that do not fill the last tile and one, two and three
256-wide K windows; the grouped call covers an empty segment and segments that
start inside a tile.  The operands are random code bytes (every E2M1 value,
both zeros), scale bytes across the normal and subnormal E4M3 range (zero
included) and tensor scales that are not powers of two."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from tests.parity import assert_gemm_close
from mean_residual_quantized_amd import averis as av

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def operand(g, rows, cols, s_dec, nseg=1):
    """Random NVFP4 bytes; returns (device tensor, list of oracle dicts per
    segment row range given later) -- here the whole-tensor bytes."""
    codes = g.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    # mostly normal scales, some subnormal and zero ones
    scales = g.integers(0x28, 0x58, size=(rows, cols // 16), dtype=np.uint8)
    sub = g.random(size=scales.shape) < 0.05
    scales[sub] = g.integers(0x00, 0x08, size=int(sub.sum()), dtype=np.uint8)
    t = av.NVFP4.empty(rows, cols, nseg, "cuda")
    t.codes.copy_(torch.from_numpy(codes))
    t.scales.copy_(torch.from_numpy(scales))
    ts = np.array([[1.0 / s, s] for s in np.atleast_1d(s_dec)], dtype=np.float32).reshape(-1)
    t.tscale.copy_(torch.from_numpy(ts))
    return t, codes, scales


def q(codes, scales, s_dec):
    return dict(codes=codes, scales=scales, s_dec=np.float32(s_dec))


# (rows, cols of the output, K): tile widths 4 (rows 16284: 64 row tiles of
# 256, 4 column tiles), 3 (32 x 8 tiles of 192 columns, the last one ragged)
# and 2 (a few tiles)
SHAPES = {
    "tile256": (16284, 1024, 256),
    "tile192": (8155, 1496, 512),
    "tile128": (1000, 208, 768),
}


@pytest.mark.parametrize("case", list(SHAPES))
def test_rank1_vanilla_and_mean_products(case):
    m, n, k = SHAPES[case]
    print("%s: m %d n %d k %d" % (case, m, n, k), flush=True)
    g = np.random.default_rng(7)
    sa, sb, sm = 0.7368421, 1.3125, 0.40625
    a, ac, asc = operand(g, m, k, sa)
    b, bc, bsc = operand(g, n, k, sb)
    mean, mc, msc = operand(g, 1, k, sm)
    qa, qb, qm = q(ac, asc, sa), q(bc, bsc, sb), q(mc, msc, sm)
    rho = torch.from_numpy(g.standard_normal(n).astype(np.float32) * 4.0)
    ab = orc.gemm(qa, qb)
    ab_bound = orc.gemm_abs_bound(qa, qb)
    rho64 = rho.numpy().astype(np.float64)
    # rank-one row given, fp32 and bf16 output
    for dt in (torch.float32, torch.bfloat16):
        c = av.averis_gemm_rank1(a, rho.cuda(), b, out_dtype=dt)
        assert_gemm_close(c, ab + rho64[None, :], ab_bound + np.abs(rho64)[None, :],
                          bf16=dt == torch.bfloat16, label="%s rank1 %s" % (case, dt))
    # vanilla
    c = av.averis_gemm_vanilla(a, b, out_dtype=torch.float32)
    assert_gemm_close(c, ab, ab_bound, label="%s vanilla" % case)
    # with a quantized mean: its rank-one term from the GEMV
    c = av.averis_gemm_fwd(a, mean, b, out_dtype=torch.float32)
    assert_gemm_close(c, orc.gemm(qa, qb, qm), orc.gemm_abs_bound(qa, qb, qm),
                      label="%s with mean" % case)
    torch.cuda.synchronize()


def test_grouped_rank1_segments():
    # three segments over 1200 rows, the middle one empty, the last one
    # starting inside a 256-row tile; each segment its own B and tensor scales
    g = np.random.default_rng(11)
    offs = np.array([0, 300, 300, 1200], dtype=np.int64)
    nseg, n, k = 3, 208, 512
    sa = np.array([0.75, 1.5, 0.3125], dtype=np.float32)
    sb = np.array([1.25, 0.5625, 2.0], dtype=np.float32)
    a, ac, asc = operand(g, int(offs[-1]), k, sa, nseg)
    b, bc, bsc = operand(g, nseg * n, k, sb, nseg)
    rho = g.standard_normal(nseg * n).astype(np.float32)
    offs_t = torch.from_numpy(offs).cuda()
    for dt in (torch.float32, torch.bfloat16):
        c = av.averis_gemm_grouped_rank1(a, torch.from_numpy(rho).cuda(), b, offs_t, out_dtype=dt)
        c = c.float().cpu().numpy()
        for s in range(nseg):
            r0, r1 = int(offs[s]), int(offs[s + 1])
            if r1 == r0:
                continue
            qa = q(ac[r0:r1], asc[r0:r1], sa[s])
            qb = q(bc[s * n:(s + 1) * n], bsc[s * n:(s + 1) * n], sb[s])
            r = rho[s * n:(s + 1) * n].astype(np.float64)
            assert_gemm_close(c[r0:r1], orc.gemm(qa, qb) + r[None, :],
                              orc.gemm_abs_bound(qa, qb) + np.abs(r)[None, :],
                              bf16=dt == torch.bfloat16, label="segment %d %s" % (s, dt))
    torch.cuda.synchronize()


def test_repeat_is_bitwise_and_matches_a_fresh_output_buffer():
    # the same call twice into buffers of different contents: identical bits
    m, n, k = SHAPES["tile192"]
    g = np.random.default_rng(3)
    a, _, _ = operand(g, m, k, 0.5)
    b, _, _ = operand(g, n, k, 1.75)
    rho = torch.from_numpy(g.standard_normal(n).astype(np.float32)).cuda()
    c1 = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    c2 = torch.zeros((m, n), dtype=torch.bfloat16, device="cuda")
    av.averis_gemm_rank1(a, rho, b, out_dtype=torch.bfloat16, out=c1)
    av.averis_gemm_rank1(a, rho, b, out_dtype=torch.bfloat16, out=c2)
    assert torch.equal(c1, c2)


# more tiles than CUs (two or more rounds of workgroups), bf16 output: full
# 256 x 256 tiles, ragged rows and columns at another tile width, and an
# output row stride that rules out 16-byte stores
ROUND_SHAPES = {
    "full": (16384, 2048, 256, 0),
    "ragged": (16400, 1040, 512, 0),
    "strided": (8448, 2048, 256, 4),
}


@pytest.mark.parametrize("case", list(ROUND_SHAPES))
def test_multi_round_bf16(case):
    m, n, k, pad = ROUND_SHAPES[case]
    print("%s: m %d n %d k %d ldc %d" % (case, m, n, k, n + pad), flush=True)
    g = np.random.default_rng(17)
    sa, sb = 0.6875, 1.4375
    a, ac, asc = operand(g, m, k, sa)
    b, bc, bsc = operand(g, n, k, sb)
    qa, qb = q(ac, asc, sa), q(bc, bsc, sb)
    rho = torch.from_numpy(g.standard_normal(n).astype(np.float32) * 4.0)
    rho64 = rho.numpy().astype(np.float64)
    ab = orc.gemm(qa, qb)
    ab_bound = orc.gemm_abs_bound(qa, qb)
    buf = torch.full((m, n + pad), float("nan"), dtype=torch.bfloat16, device="cuda")
    c = buf[:, :n]
    av.averis_gemm_rank1(a, rho.cuda(), b, out_dtype=torch.bfloat16, out=c)
    assert_gemm_close(c, ab + rho64[None, :], ab_bound + np.abs(rho64)[None, :], bf16=True,
                      label="%s rank1" % case)
    # the fp32 output holds the same values before rounding: the bf16 output
    # is their round-to-nearest-even, bit for bit
    c32 = av.averis_gemm_rank1(a, rho.cuda(), b, out_dtype=torch.float32)
    assert torch.equal(c, c32.to(torch.bfloat16))
    if pad:
        assert torch.isnan(buf[:, n:].float()).all()     # nothing past the row
    cv = av.averis_gemm_vanilla(a, b, out_dtype=torch.bfloat16)
    assert_gemm_close(cv, ab, ab_bound, bf16=True, label="%s vanilla" % case)
    assert torch.equal(cv, av.averis_gemm_vanilla(a, b, out_dtype=torch.float32).to(torch.bfloat16))
    torch.cuda.synchronize()
