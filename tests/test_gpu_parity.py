"""GPU parity: libaveris (through the C ABI) against the CPU oracle.

Quantized codes, scale bytes, tensor scales and the fp32 mean must be
bit-exact; GEMM outputs must satisfy both
    |C_gpu - C_oracle| <= 1e-3 * (|deq A| |deq B|^T + 1 |deq mean| |deq B|^T)
elementwise and max |C_gpu - C_oracle| <= 1e-3 max |C_oracle| (tests/parity.py),
where C_oracle is the oracle's float64 product of the same dequantized
operands (an FP32-accumulated product of exact operands meets the first with
a wide margin: K * 2^-24 < 2e-4 at K = 3072).  Full-size workloads are in
test_gpu_fullsize.py."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from tests.parity import assert_gemm_close, assert_quant_equal
from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def f32(t):
    return t.float().cpu().numpy()


def quant_weights(w, rnd=av.RN):
    return (av.averis_quant(w, transpose=True, rnd=rnd, sr_stream=av.STREAM_WEIGHT),
            av.averis_quant(w, transpose=False, rnd=rnd, sr_stream=av.STREAM_WEIGHT))


def full_check(x, w, d, seed=0, rnd="sr"):
    """Split-quant of X and D, weight quant, fwd/dgrad/vanilla GEMMs vs oracle."""
    r = av.SR if rnd == "sr" else av.RN
    xg, wg, dg = x.cuda(), w.cuda(), d.cuda()
    xn, wn, dn = f32(x), f32(w), f32(d)

    wt_g, wd_g = quant_weights(wg)
    wq = orc.weight_quant(wn, "rn")
    assert_quant_equal(wt_g, wq["fwd"])
    assert_quant_equal(wd_g, wq["dgrad"])

    for a_g, a_n, b_g, b_ref, fn in [(xg, xn, wt_g, wq["fwd"], av.averis_gemm_fwd),
                                     (dg, dn, wd_g, wq["dgrad"], av.averis_gemm_dgrad)]:
        res, mean, mu = av.averis_split_quant(a_g, seed=seed, rnd=r)
        s = orc.split_quant(a_n, rnd, seed)
        np.testing.assert_array_equal(mu.cpu().numpy(), s["mu"])
        assert_quant_equal(res, s["residual"])
        assert_quant_equal(mean, s["mean"])
        c = fn(res, mean, b_g)
        ref = orc.gemm(s["residual"], b_ref, s["mean"])
        assert_gemm_close(c, ref, orc.gemm_abs_bound(s["residual"], b_ref, s["mean"]))

    # vanilla arm (forward)
    qv = av.averis_quant(xg, seed=seed, rnd=r)
    qv_ref = orc.vanilla_quant(xn, rnd, seed)
    assert_quant_equal(qv, qv_ref)
    c = av.averis_gemm_vanilla(qv, wt_g)
    assert_gemm_close(c, orc.gemm(qv_ref, wq["fwd"]), orc.gemm_abs_bound(qv_ref, wq["fwd"]))
    torch.cuda.synchronize()


def test_tiny():
    cfg = workloads.tiny()
    full_check(cfg["x"], cfg["w"], cfg["d"], seed=0)


def test_tiny_round_to_nearest_and_other_seed():
    cfg = workloads.tiny()
    full_check(cfg["x"], cfg["w"], cfg["d"], seed=0, rnd="rn")
    full_check(cfg["x"], cfg["w"], cfg["d"], seed=0xABCDEF0123456789)


def test_ragged_shapes_several_tiles():
    # rows not a multiple of any chunk or tile; cols not a multiple of the
    # 512/1024-column tiles; N not a multiple of the 128-wide GEMM tile
    cfg = workloads.up_proj(l=1000, m=304, n=208)
    full_check(cfg["x"], cfg["w"], cfg["d"], seed=7)


def test_ragged_rows_and_cols_fast_gemm_path():
    # K % 64 == 0 in both passes (the fast GEMM kernel) with M and N tails
    cfg = workloads.up_proj(l=1000, m=320, n=192)
    full_check(cfg["x"], cfg["w"], cfg["d"], seed=11)


def test_swiglu_shapes_reduced():
    cfg = workloads.down_proj(l=520, m=3072, n=1024)
    full_check(cfg["x"], cfg["w"], cfg["d"], seed=3)


def test_single_block_and_single_row():
    rng = np.random.default_rng(0)
    for rows, cols in [(1, 16), (3, 16), (1, 64), (200, 16)]:
        x = torch.from_numpy((rng.standard_normal((rows, cols)) * 2 + 1).astype(np.float32))
        w = torch.from_numpy((rng.standard_normal((cols, 32)) / 4).astype(np.float32))
        d = torch.from_numpy(rng.standard_normal((rows, 32)).astype(np.float32))
        full_check(x, w, d, seed=rows)


def test_constant_columns_give_zero_residual_and_mean_rows():
    mu = (3 * np.random.default_rng(1).standard_normal(128) + 1.5).astype(np.float32)
    x = torch.from_numpy(np.tile(mu, (77, 1))).to(torch.bfloat16)
    res, mean, m = av.averis_split_quant(x.cuda(), seed=5)
    s = orc.split_quant(f32(x), "sr", 5)
    assert_quant_equal(res, s["residual"])
    assert_quant_equal(mean, s["mean"])
    g = res.cpu()
    assert g["tscale"][0] == 1 and not (g["codes"] & 0x77).any()


def test_all_zero_and_empty_inputs():
    z = torch.zeros((40, 64), dtype=torch.bfloat16, device="cuda")
    res, mean, mu = av.averis_split_quant(z, seed=1)
    assert not res.codes.any() and not res.scales.any() and not mean.codes.any()
    assert res.tscale.tolist() == [1.0, 1.0] and mean.tscale.tolist() == [1.0, 1.0]
    e = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    res, mean, mu = av.averis_split_quant(e, seed=1)
    assert res.codes.numel() == 0 and not mu.any() and mean.tscale.tolist() == [1.0, 1.0]
    q = av.averis_quant(e)
    assert q.tscale.tolist() == [1.0, 1.0]
    torch.cuda.synchronize()


def adversarial_columns(rows, cols, seed):
    """Columns whose fp64 running sum is order-dependent (the kernel's
    exactness certificate fails for them and the exact sum is taken)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    i = np.arange(rows)
    x[:, 0] = np.resize(np.array([2.0 ** 100, 1.0, -(2.0 ** 100)], np.float32), rows)
    x[:, 1] = np.where(i % 2 == 0, np.float32(3.0e30), np.float32(-1.0e-30))
    x[:, 2] = np.where(i % 5 == 0, np.float32(7.0), np.float32(2.0 ** -130))   # fp32 subnormal
    x[:, 3] = 0.0
    x[:, 5] = np.where(i % 3 == 0, np.float32(2.0 ** 60), np.float32(0.75)) * np.where(i % 2, 1, -1)
    # chunks of 128 rows that are each exact on their own while the column as
    # a whole is not: tiny values in the first chunk, huge ones after it (the
    # exact sum then adds the chunks' exact partials)
    small = rng.integers(-100, 100, rows) * np.float32(2.0 ** -60)
    large = rng.integers(-100, 100, rows) * np.float32(2.0 ** 40)
    x[:, 6] = np.where(i < 128, small, large).astype(np.float32)
    x[:, 7] = np.where((i // 128) % 2 == 0, large, small).astype(np.float32)
    # not certified, but every value on one grid narrow enough for an exact
    # 64-bit sum in its units (column 8 as bf16, column 9 as fp32): the
    # fallback's integer path, with a total that needs rounding to a double
    k = rng.integers(1, 65, rows).astype(np.float32)
    m = rng.integers(129, 256, rows).astype(np.float32) * np.where(i % 2, 1, -1)
    x[:, 8] = np.where(i % 7 == 0, k * np.float32(2.0 ** 12), m * np.float32(2.0 ** -29))
    x[:, 9] = np.where(i % 7 == 0, k * np.float32(2.0 ** 10),
                       ((0.5 + rng.random(rows) / 2) * 2.0 ** -8 * np.where(i % 2, 1, -1)).astype(np.float32))
    return x


@pytest.mark.parametrize("rows", [300, 4000])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_uncertified_columns_take_the_exact_sum(dtype, rows):
    x = torch.from_numpy(adversarial_columns(rows, 64, 5)).to(dtype)
    res, mean, mu = av.averis_split_quant(x.cuda(), seed=3)
    s = orc.split_quant(f32(x), "sr", 3)
    np.testing.assert_array_equal(mu.cpu().numpy(), s["mu"])
    assert_quant_equal(res, s["residual"])
    assert_quant_equal(mean, s["mean"])
    # grouped: each segment's mean on its own rows
    offs = np.array([0, 97, 97, rows], dtype=np.int64)
    og = torch.from_numpy(offs).cuda()
    res_g, mean_g, mu_g = av.averis_split_quant_grouped(x.cuda(), og, seed=3)
    g = orc.split_quant_grouped(f32(x), offs, "sr", 3)
    np.testing.assert_array_equal(mu_g.cpu().numpy(), g["mu"])
    rc = res_g.cpu()
    for seg in range(3):
        r0, r1 = offs[seg], offs[seg + 1]
        np.testing.assert_array_equal(rc["codes"][r0:r1], g["residual"][seg]["codes"])
        assert rc["tscale"][2 * seg] == g["residual"][seg]["s_enc"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_uncertified_columns_in_many_short_segments(dtype):
    # nine segments (two empty) over 2000 rows: the finalize for short
    # segments takes four segments per workgroup, so the columns that fail the
    # certificate sit in segments of the second and third workgroup rows and
    # in waves other than the first; 130 columns leave a ragged last tile
    rows, cols = 2000, 130 + 14
    x = adversarial_columns(rows, cols, 9)
    x[:, 64:72] = x[:, 0:8]            # failing columns in the second 64-column tile too
    x = torch.from_numpy(x).to(dtype)
    offs = np.array([0, 100, 100, 350, 700, 700, 900, 1300, 1500, 2000], dtype=np.int64)
    nseg = len(offs) - 1
    res_g, mean_g, mu_g = av.averis_split_quant_grouped(x.cuda(), torch.from_numpy(offs).cuda(),
                                                        seed=4)
    g = orc.split_quant_grouped(f32(x), offs, "sr", 4)
    np.testing.assert_array_equal(mu_g.cpu().numpy(), g["mu"])
    rc, mc = res_g.cpu(), mean_g.cpu()
    for seg in range(nseg):
        r0, r1 = offs[seg], offs[seg + 1]
        print("segment %d rows %d..%d" % (seg, r0, r1), flush=True)
        np.testing.assert_array_equal(rc["codes"][r0:r1], g["residual"][seg]["codes"])
        np.testing.assert_array_equal(rc["scales"][r0:r1], g["residual"][seg]["scales"])
        assert rc["tscale"][2 * seg] == g["residual"][seg]["s_enc"]
        np.testing.assert_array_equal(mc["codes"][seg], g["mean"][seg]["codes"][0])
        np.testing.assert_array_equal(mc["scales"][seg], g["mean"][seg]["scales"][0])
        assert mc["tscale"][2 * seg] == g["mean"][seg]["s_enc"]


def test_bf16_output_within_rounding():
    cfg = workloads.up_proj(l=256, m=256, n=128)
    xg = cfg["x"].cuda()
    wt_g, _ = quant_weights(cfg["w"].cuda())
    res, mean, _ = av.averis_split_quant(xg, seed=0)
    y32 = av.averis_gemm_fwd(res, mean, wt_g, out_dtype=torch.float32)
    y16 = av.averis_gemm_fwd(res, mean, wt_g, out_dtype=torch.bfloat16)
    torch.testing.assert_close(y16, y32.to(torch.bfloat16), rtol=0, atol=0)


@pytest.mark.parametrize("l,m,n", [(1000, 320, 192), (520, 1024, 208), (8192, 1024, 3072)])
def test_bf16_output_edges_and_strides(l, m, n):
    # bf16 output leaves through an LDS-staged tile: full 16-byte pieces go out
    # as one store, pieces past the tile's edge or in rows that are not
    # 16-byte aligned element by element; both must equal fp32 -> bf16 (RNE)
    cfg = workloads.up_proj(l=l, m=m, n=n)
    xg, dg = cfg["x"].cuda(), cfg["d"].cuda()
    wt_g, wd_g = quant_weights(cfg["w"].cuda())
    for a_g, b_g, fn, cols in [(xg, wt_g, av.averis_gemm_fwd, n), (dg, wd_g, av.averis_gemm_dgrad, m)]:
        res, mean, _ = av.averis_split_quant(a_g, seed=4)
        y32 = fn(res, mean, b_g, out_dtype=torch.float32)
        ref = y32.to(torch.bfloat16)
        y16 = fn(res, mean, b_g, out_dtype=torch.bfloat16)
        assert torch.equal(y16, ref)
        # row stride cols + 3 (odd) and a base 2 bytes past 16-byte alignment
        big = torch.zeros((l, cols + 8), dtype=torch.bfloat16, device="cuda")
        view = big.view(-1)[1:1 + l * (cols + 3)].view(l, cols + 3)[:, :cols]
        fn(res, mean, b_g, out_dtype=torch.bfloat16, out=view)
        assert torch.equal(view, ref)
        v16 = av.averis_gemm_vanilla(res, b_g, out_dtype=torch.bfloat16)
        assert torch.equal(v16, av.averis_gemm_vanilla(res, b_g, out_dtype=torch.float32).to(torch.bfloat16))
    torch.cuda.synchronize()


def test_deterministic_repeats():
    cfg = workloads.up_proj(l=512, m=256, n=128)
    xg = cfg["x"].cuda()
    outs = [av.averis_split_quant(xg, seed=9) for _ in range(3)]
    for r, m, mu in outs[1:]:
        assert torch.equal(r.codes, outs[0][0].codes) and torch.equal(r.scales, outs[0][0].scales)
        assert torch.equal(m.codes, outs[0][1].codes) and torch.equal(mu, outs[0][2])


@pytest.mark.parametrize("l,m,n", [(1000, 320, 192), (300, 64, 128), (256, 128, 64),
                                   (8192, 1024, 3072)])
def test_gemm_bitwise_repeatable(l, m, n):
    # Regression: on the exit path of the K loop the epilogue read the last
    # MFMA's accumulator before it completed (missing wait states); results
    # then varied between runs.  Repeated runs must agree bit for bit, and
    # with the oracle.
    cfg = workloads.up_proj(l=l, m=m, n=n)
    wt, wd = quant_weights(cfg["w"].cuda())
    xr, xm, _ = av.averis_split_quant(cfg["x"].cuda(), seed=3)
    dr, dm, _ = av.averis_split_quant(cfg["d"].cuda(), seed=4)
    for fn, a, mu, b in [(av.averis_gemm_fwd, xr, xm, wt), (av.averis_gemm_dgrad, dr, dm, wd)]:
        outs = [fn(a, mu, b, out_dtype=torch.float32) for _ in range(5)]
        for o in outs[1:]:
            assert torch.equal(o, outs[0])
        vo = [av.averis_gemm_vanilla(a, b, out_dtype=torch.bfloat16) for _ in range(3)]
        for o in vo[1:]:
            assert torch.equal(o, vo[0])
    if l <= 1000:
        wq = orc.weight_quant(f32(cfg["w"]), "rn")
        s = orc.split_quant(f32(cfg["d"]), "sr", 4)
        c = av.averis_gemm_dgrad(dr, dm, wd, out_dtype=torch.float32)
        assert_gemm_close(c, orc.gemm(s["residual"], wq["dgrad"], s["mean"]),
                          orc.gemm_abs_bound(s["residual"], wq["dgrad"], s["mean"]))


def test_grouped_moe_reduced():
    cfg = workloads.moe(tokens=256, topk=8, experts=16, hidden=128, inter=64)
    x, w, d, offs = cfg["x"], cfg["w"], cfg["d"], cfg["offsets"]
    nseg = len(offs) - 1
    og = torch.from_numpy(offs).cuda()
    xn, wn = f32(x), f32(w)
    res, mean, mu = av.averis_split_quant_grouped(x.cuda(), og, seed=2)
    g = orc.split_quant_grouped(xn, offs, "sr", 2)
    np.testing.assert_array_equal(mu.cpu().numpy(), g["mu"])
    rc = res.cpu()
    for s in range(nseg):
        r0, r1 = offs[s], offs[s + 1]
        np.testing.assert_array_equal(rc["codes"][r0:r1], g["residual"][s]["codes"])
        np.testing.assert_array_equal(rc["scales"][r0:r1], g["residual"][s]["scales"])
        assert rc["tscale"][2 * s] == g["residual"][s]["s_enc"]
        assert rc["tscale"][2 * s + 1] == g["residual"][s]["s_dec"]
        mc = mean.cpu()
        np.testing.assert_array_equal(mc["codes"][s:s + 1], g["mean"][s]["codes"])
        assert mc["tscale"][2 * s] == g["mean"][s]["s_enc"]
    # per-expert weights, forward copies
    wt = av.averis_quant_batched(w.cuda(), transpose=True)
    wrefs = [orc.weight_quant(wn[e], "rn")["fwd"] for e in range(nseg)]
    wc = wt.cpu()
    n = w.shape[2]
    for e in range(nseg):
        np.testing.assert_array_equal(wc["codes"][e * n:(e + 1) * n], wrefs[e]["codes"])
        assert wc["tscale"][2 * e + 1] == wrefs[e]["s_dec"]
    y = av.averis_gemm_grouped(res, mean, wt, og)
    ref = orc.gemm_grouped(g["residual"], wrefs, g["mean"])
    bound = np.concatenate([orc.gemm_abs_bound(g["residual"][s], wrefs[s], g["mean"][s])
                            for s in range(nseg)])
    assert_gemm_close(y, ref, bound)
    # vanilla grouped
    qv = av.averis_quant_grouped(x.cuda(), og, seed=2)
    vrefs = orc.vanilla_quant_grouped(xn, offs, "sr", 2)
    qc = qv.cpu()
    for s in range(nseg):
        np.testing.assert_array_equal(qc["codes"][offs[s]:offs[s + 1]], vrefs[s]["codes"])
        assert qc["tscale"][2 * s] == vrefs[s]["s_enc"]
    yv = av.averis_gemm_grouped(qv, None, wt, og)
    assert_gemm_close(yv, orc.gemm_grouped(vrefs, wrefs),
                      np.concatenate([orc.gemm_abs_bound(vrefs[s], wrefs[s]) for s in range(nseg)]))


def test_workspace_reused_across_calls():
    # the workspace holds intermediate results only: one workspace per shape
    # serves many calls in a row (the plain, ratio and rank-one forms of the
    # split, plain quant in between; the grouped split with plain grouped
    # quant) and every result equals the result of a fresh workspace.
    rows, cols = 1000, 320
    cfg = workloads.up_proj(l=rows, m=cols, n=192)
    offs = torch.tensor([0, 100, 100, 999, 1000], dtype=torch.int64, device="cuda")
    nseg = offs.numel() - 1
    filled = lambda n: torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    ws1 = filled(max(av.workspace_bytes(av.OP_SPLIT_QUANT, rows, cols),
                    av.workspace_bytes(av.OP_QUANT, rows, cols)))
    wsg = filled(max(av.workspace_bytes(av.OP_SPLIT_QUANT, rows, cols, 0, nseg),
                    av.workspace_bytes(av.OP_QUANT, rows, cols, 0, nseg)))
    wq = av.averis_quant(cfg["w"].cuda(), transpose=True, rnd=av.RN, sr_stream=av.STREAM_WEIGHT)
    flat = lambda outs: [t for o in outs for t in ((o.codes, o.scales, o.tscale)
                                                   if isinstance(o, av.NVFP4) else (o,))]
    for it in range(4):
        x = (cfg["x"].float() * (1 + it) + it).to(torch.bfloat16).cuda()
        runs = [
            (ws1, lambda w: av.averis_split_quant(x, seed=it, ws=w)),
            (ws1, lambda w: (av.averis_quant(x, seed=it, ws=w),)),
            (ws1, lambda w: av.averis_split_quant_ratio(x, seed=it, ws=w)),
            (ws1, lambda w: av.averis_split_quant_rank1(x, wq, seed=it, ws=w)),
            (wsg, lambda w: av.averis_split_quant_grouped(x, offs, seed=it, ws=w)),
            (wsg, lambda w: (av.averis_quant_grouped(x, offs, seed=it, ws=w),)),
            (wsg, lambda w: av.averis_split_quant_ratio(x, seed=it, offsets=offs, ws=w)),
        ]
        for ws, run in runs:
            got = flat(run(ws))
            ref = flat(run(None))            # a fresh workspace
            for g, r in zip(got, ref):
                assert torch.equal(g, r)
    torch.cuda.synchronize()
