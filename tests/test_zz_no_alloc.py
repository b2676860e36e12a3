"""The allocation-free split-quant (averis_split_quant_noalloc, whose
workspace is the library's own device array) through the C ABI, against
averis_split_quant with a workspace of its own: bit for bit on two calls in a
row, the second on a smaller input (the array keeps the first call's
contents), and on a third call in fp32."""

import pytest
import torch

from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def same_as_workspace_call(a, seed, rnd):
    print("noalloc split: %s %s, seed %d" % (tuple(a.shape), a.dtype, seed), flush=True)
    got = av.averis_split_quant_noalloc(a, seed=seed, rnd=rnd)
    ref = av.averis_split_quant(a, seed=seed, rnd=rnd)
    for g, r in zip(got[:2], ref[:2]):
        for t in ("codes", "scales", "tscale"):
            assert torch.equal(getattr(g, t), getattr(r, t)), t
    assert torch.equal(got[2], ref[2])


def test_two_calls_in_a_row_the_second_smaller():
    big = workloads.block_linear("gate")["d"]          # 16384 x 3072 bf16, the largest D
    same_as_workspace_call(big.cuda(), seed=1, rnd=av.SR)
    small = workloads.up_proj(l=1000, m=320, n=208)["x"]
    same_as_workspace_call(small.cuda(), seed=4, rnd=av.SR)
    tiny = workloads.tiny()["x"]                         # 64 x 128 fp32
    same_as_workspace_call(tiny.cuda(), seed=0, rnd=av.RN)
    torch.cuda.synchronize()


def test_too_large_is_rejected_before_any_launch():
    rows, cols = 32768, 3072
    a = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(av.AverisError) as e:
        av.averis_split_quant_noalloc(a, seed=0)
    assert e.value.status == 5
    torch.cuda.synchronize()
