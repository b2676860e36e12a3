"""GPU parity of the mean-energy ratio R = ||mu|| / sqrt(||A||_F^2 / l) that
averis_split_quant_ratio computes alongside the split (against the oracle's
float64 value from exact sums; the GPU sums in fp64 in another order and
rounds R to fp32, so the bar is 1e-6 relative), and bit-equality of its
quantized outputs with averis_split_quant."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads

pytestmark = pytest.mark.gpu

RTOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def close(r_gpu, r_ref):
    assert abs(float(r_gpu) - r_ref) <= RTOL * abs(r_ref) + 1e-12, (float(r_gpu), r_ref)


def same_split(a_g, seed=0):
    res, mean, mu, ratio = av.averis_split_quant_ratio(a_g, seed=seed)
    r2, m2, mu2 = av.averis_split_quant(a_g, seed=seed)
    for x, y in ((res, r2), (mean, m2)):
        for t in ("codes", "scales", "tscale"):
            assert torch.equal(getattr(x, t), getattr(y, t)), t
    assert torch.equal(mu, mu2)
    return ratio


@pytest.mark.parametrize("which", ["x", "d"])
def test_tiny(which):
    a = workloads.tiny()[which]
    ratio = same_split(a.cuda())
    close(ratio[0], orc.mean_energy_ratio(a.float().numpy()))


@pytest.mark.parametrize("l,m", [(2048, 320), (1000, 208), (1, 64), (129, 16)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_shapes(l, m, dtype):
    rng = np.random.default_rng(l + m)
    a = rng.standard_normal((l, m)) * 0.5 + (3 * rng.standard_normal(m) + 1.5)[None, :]
    t = torch.from_numpy(a.astype(np.float32)).to(dtype)
    ratio = same_split(t.cuda(), seed=l)
    close(ratio[0], orc.mean_energy_ratio(t.float().numpy()))


@pytest.mark.parametrize("which", ["x", "d"])
def test_full_size_up_proj(which):
    a = workloads.up_proj()[which]
    ratio = same_split(a.cuda())
    close(ratio[0], orc.mean_energy_ratio(a.float().numpy()))


def test_degenerate_inputs():
    mu = torch.randn(96) * 3
    r = av.averis_split_quant_ratio(mu.repeat(40, 1).cuda())[3]
    close(r[0], 1.0)
    assert av.averis_split_quant_ratio(torch.zeros((64, 32), device="cuda"))[3].item() == 0.0
    assert av.averis_split_quant_ratio(torch.zeros((0, 32), device="cuda"))[3].item() == 0.0


def test_grouped_with_an_empty_segment():
    cfg = workloads.moe(tokens=256, topk=8, experts=16, hidden=128, inter=64)
    x, offs = cfg["x"], np.array(cfg["offsets"], dtype=np.int64)
    x = torch.cat([x[:offs[2]], x[offs[3]:]])     # drop segment 2's rows: it is empty
    offs[3:] -= offs[3] - offs[2]
    offs_g = torch.from_numpy(offs).cuda()
    res, mean, mu, ratio = av.averis_split_quant_ratio(x.cuda(), seed=4, offsets=offs_g)
    r2, m2, mu2 = av.averis_split_quant_grouped(x.cuda(), offs_g, seed=4)
    for a, b in ((res, r2), (mean, m2)):
        for t in ("codes", "scales", "tscale"):
            assert torch.equal(getattr(a, t), getattr(b, t)), t
    ref = orc.mean_energy_ratio_grouped(x.float().numpy(), offs)
    assert ratio[2].item() == 0.0 and ref[2] == 0.0
    for s in range(len(ref)):
        close(ratio[s], ref[s])
