"""GPU parity of averis_quant_pair (both quantized copies of a weight in one
call) against the oracle's weight quantization, and against the one-copy
entry points, bit for bit."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def same(gpu, ref, rows=None, seg=0):
    g = gpu.cpu()
    codes, scales = g["codes"], g["scales"]
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    np.testing.assert_array_equal(codes, ref["codes"])
    np.testing.assert_array_equal(scales, ref["scales"])
    assert g["tscale"][2 * seg] == ref["s_enc"] and g["tscale"][2 * seg + 1] == ref["s_dec"]


def same_gpu(a, b):
    for t in ("codes", "scales", "tscale"):
        assert torch.equal(getattr(a, t), getattr(b, t)), t


@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_full_size_weight_matches_oracle_and_one_copy_calls(rnd):
    w = workloads.up_proj()["w"]                 # 1024 x 3072 bf16
    r = av.RN if rnd == "rn" else av.SR
    wg = w.cuda()
    wt, wd = av.averis_quant_pair(wg, seed=3, rnd=r)
    ref = orc.weight_quant(w.float().numpy(), rnd, 3)
    same(wt, ref["fwd"])
    same(wd, ref["dgrad"])
    same_gpu(wt, av.averis_quant(wg, transpose=True, seed=3, rnd=r, sr_stream=av.STREAM_WEIGHT))
    same_gpu(wd, av.averis_quant(wg, transpose=False, seed=3, rnd=r, sr_stream=av.STREAM_WEIGHT))


@pytest.mark.parametrize("rows,cols", [(304, 208), (16, 16), (64, 64), (80, 1040), (2000, 48)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_tiles_and_dtypes(rows, cols, dtype):
    rng = np.random.default_rng(rows * 7 + cols)
    w = torch.from_numpy((rng.standard_normal((rows, cols)) * 0.05).astype(np.float32)).to(dtype)
    wn = w.float().numpy()
    for rnd, r in (("rn", av.RN), ("sr", av.SR)):
        wt, wd = av.averis_quant_pair(w.cuda(), seed=rows, rnd=r)
        ref = orc.weight_quant(wn, rnd, rows)
        same(wt, ref["fwd"])
        same(wd, ref["dgrad"])


def test_row_stride_and_batch_of_experts():
    rng = np.random.default_rng(11)
    e, m, n = 3, 128, 96
    big = torch.from_numpy(rng.standard_normal((e, m, n + 32)).astype(np.float32)).to(torch.bfloat16)
    w = big.cuda()[:, :, :n]                     # row stride n + 32, batch stride m (n + 32)
    wt, wd = av.averis_quant_pair(w, seed=9, rnd=av.SR)
    wn = big[:, :, :n].float().numpy()
    for b in range(e):
        rt = orc.quantize(np.ascontiguousarray(wn[b].T), "sr", 9, stream=2, row0=b * n)
        rd = orc.quantize(wn[b], "sr", 9, stream=2, row0=b * m)
        same(wt, rt, rows=slice(b * n, (b + 1) * n), seg=b)
        same(wd, rd, rows=slice(b * m, (b + 1) * m), seg=b)
    same_gpu(wt, av.averis_quant_batched(w, transpose=True, seed=9, rnd=av.SR))
    same_gpu(wd, av.averis_quant_batched(w, transpose=False, seed=9, rnd=av.SR))


def test_zero_weight():
    w = torch.zeros((32, 48), dtype=torch.bfloat16, device="cuda")
    wt, wd = av.averis_quant_pair(w)
    for q in (wt, wd):
        assert not q.codes.any() and not q.scales.any()
        assert q.tscale.tolist() == [1.0, 1.0]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_multi_weight_call_matches_oracle_and_single_calls(dtype, rnd):
    """averis_quant_pair_multi: each weight's two copies equal the oracle's and
    averis_quant_pair's with that weight's seed, over shapes of their own
    (ragged 64 x 64 tiles, one weight with a row stride above its width)."""
    rng = np.random.default_rng(5)
    r = av.RN if rnd == "rn" else av.SR
    shapes = [(304, 208), (16, 16), (80, 1040), (2000, 48), (128, 96)]
    ws_cpu = [torch.from_numpy((rng.standard_normal(s) * 0.05 * (i + 1)).astype(np.float32))
              .to(dtype) for i, s in enumerate(shapes)]
    wg = [w.cuda() for w in ws_cpu]
    wide = torch.zeros((128, 96 + 32), dtype=dtype, device="cuda")
    wide[:, :96] = wg[4]
    wg[4] = wide[:, :96]                         # row stride 128
    seeds = [3, 11, 0, 7, 2 ** 40 + 5]
    outs = av.averis_quant_pair_multi(wg, seeds=seeds, rnd=r)
    for i, (w, (wt, wd)) in enumerate(zip(wg, outs)):
        ref = orc.weight_quant(ws_cpu[i].float().numpy(), rnd, seeds[i])
        same(wt, ref["fwd"])
        same(wd, ref["dgrad"])
        st, sd = av.averis_quant_pair(w, seed=seeds[i], rnd=r)
        same_gpu(wt, st)
        same_gpu(wd, sd)


def test_multi_weight_call_block_shapes_and_repeat():
    """The seven Qwen3-0.6B-like weights in one call, twice in a row (the
    workspace's partials are rewritten, not accumulated), against the
    single-weight calls; one zero weight among them."""
    shapes = [(1024, 2048), (1024, 1024), (1024, 1024), (2048, 1024), (1024, 3072),
              (1024, 3072), (3072, 1024)]
    g = torch.Generator(device="cuda").manual_seed(1)
    wg = [(torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for s in shapes]
    wg[2].zero_()
    for _ in range(2):
        outs = av.averis_quant_pair_multi(wg, rnd=av.SR, seeds=list(range(7)))
        for i, w in enumerate(wg):
            st, sd = av.averis_quant_pair(w, seed=i, rnd=av.SR)
            same_gpu(outs[i][0], st)
            same_gpu(outs[i][1], sd)
    assert outs[2][0].tscale.tolist() == [1.0, 1.0]
