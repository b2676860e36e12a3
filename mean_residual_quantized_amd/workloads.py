"""Seeded synthetic inputs for the Averis linear (no method arithmetic here).

The pages train Qwen3-0.6B (and a 7B-A1.5B MoE) on DCLM; none of that is
available, so these generators stand in for the activations, weights and
output gradients with the structure [Lighthouse] §2.1 describes: a coherent
rank-one mean 1 mu^T, a low-rank spike U S V^T and a Gaussian tail.  Shapes
follow the Qwen3-0.6B linears (hidden 1024, intermediate 3072, q 2048).

Conventions: N(a, b) is mean a and variance b; values are drawn in float64,
rounded to float32, then to bfloat16 by torch (round-to-nearest-even).  Every
tensor has its own generator seeded by (workload, tensor id, linear id).
"""

import numpy as np
import torch

# tensor ids for the seed sequence
T_X, T_W, T_D, T_ROUTE = 0, 1, 2, 3

# the Qwen3-0.6B-like block: name -> (K_in, N_out)
QWEN3_06B_LINEARS = {
    "q": (1024, 2048), "k": (1024, 1024), "v": (1024, 1024), "o": (2048, 1024),
    "gate": (1024, 3072), "up": (1024, 3072), "down": (3072, 1024),
}


def rng_for(cfg, tensor_id, linear_id=0):
    return np.random.default_rng(np.random.SeedSequence([cfg, tensor_id, linear_id]))


def _orthonormal(rng, rows, k):
    q, r = np.linalg.qr(rng.standard_normal((rows, k)))
    return q * np.sign(np.diag(r))[None, :]


def _cast(a64, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


def mean_biased_activation(rng, l, m, mu_scale=3.0, mu_bias=1.5, spike=(4.0, 2.0, 1.0, 0.5),
                           tail_sigma=0.5, dtype=torch.bfloat16):
    """X = 1 mu^T + U diag(spike) V^T + tail; mu_j = mu_scale * z + mu_bias."""
    mu = mu_scale * rng.standard_normal(m) + mu_bias
    k = len(spike)
    u = _orthonormal(rng, l, k)
    v = _orthonormal(rng, m, k)
    x = (u * np.asarray(spike)[None, :]) @ v.T
    x += mu[None, :]
    x += tail_sigma * rng.standard_normal((l, m))
    return _cast(x, dtype)


def swiglu_activation(rng, l, m, base=0.3, off_mean=0.5, off_var=0.5, dtype=torch.bfloat16):
    """X = silu(A) * B with A, B ~ N(base + o_j, 1) and o_j ~ N(off_mean, off_var)."""
    o = off_mean + np.sqrt(off_var) * rng.standard_normal(m)
    a = base + o[None, :] + rng.standard_normal((l, m))
    b = base + o[None, :] + rng.standard_normal((l, m))
    x = a / (1.0 + np.exp(-a)) * b
    return _cast(x, dtype)


def gradient(rng, l, n, nu_sigma=0.05, noise_var=1e-3, const_mean=None, dtype=torch.bfloat16):
    """D = 1 nu^T + N(0, noise_var); nu_j ~ N(0, nu_sigma^2), or nu_j = const_mean."""
    nu = np.full(n, const_mean) if const_mean is not None else nu_sigma * rng.standard_normal(n)
    d = nu[None, :] + np.sqrt(noise_var) * rng.standard_normal((l, n))
    return _cast(d, dtype)


def weight(rng, m, n, dtype=torch.bfloat16):
    """W (m x n) ~ N(0, 1/m)."""
    return _cast(rng.standard_normal((m, n)) / np.sqrt(m), dtype)


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def tiny():
    """Tiny case: X f32 64x128 (rank-2 spike), W 128x64, D 64x64 = 0.2 + N(0,1)."""
    f32 = torch.float32
    x = mean_biased_activation(rng_for(0, T_X), 64, 128, spike=(4.0, 2.0), tail_sigma=0.5, dtype=f32)
    w = weight(rng_for(0, T_W), 128, 64, dtype=f32)
    d = gradient(rng_for(0, T_D), 64, 64, const_mean=0.2, noise_var=1.0, dtype=f32)
    return dict(x=x, w=w, d=d)


def up_proj(l=8192, m=1024, n=3072):
    """Up-proj: X bf16 l x m (mu scale 3, rank-4 spike, tail sigma 0.5), W m x n, D l x n."""
    x = mean_biased_activation(rng_for(1, T_X), l, m)
    w = weight(rng_for(1, T_W), m, n)
    d = gradient(rng_for(1, T_D), l, n)
    return dict(x=x, w=w, d=d)


def down_proj(l=8192, m=3072, n=1024):
    """Down-proj: X = silu(A) * B (positive heavy mean), W m x n, D l x n."""
    x = swiglu_activation(rng_for(2, T_X), l, m)
    w = weight(rng_for(2, T_W), m, n)
    d = gradient(rng_for(2, T_D), l, n)
    return dict(x=x, w=w, d=d)


def moe_routing(rng, tokens, experts, topk, zipf_s=1.1):
    """Row counts per expert for `tokens` tokens routed top-k without
    replacement (Gumbel-top-k) under Zipf(zipf_s) popularity p_e ~ e^-s."""
    logp = -zipf_s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    keys = logp[None, :] + rng.gumbel(size=(tokens, experts))
    chosen = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]
    counts = np.bincount(chosen.ravel(), minlength=experts)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def moe(tokens=4096, topk=8, experts=64, hidden=2048, inter=768):
    """MoE grouped case: tokens * topk routed rows sorted by expert; per-expert
    mean (scale 2) + N(0, 0.25) rows; W_e hidden x inter; D rows x inter."""
    offsets = moe_routing(rng_for(3, T_ROUTE), tokens, experts, topk)
    rows = int(offsets[-1])
    rx = rng_for(3, T_X)
    x = np.empty((rows, hidden), dtype=np.float64)
    for e in range(experts):
        r0, r1 = offsets[e], offsets[e + 1]
        mu = 2.0 * rx.standard_normal(hidden)
        x[r0:r1] = mu[None, :] + 0.5 * rx.standard_normal((r1 - r0, hidden))
    rw = rng_for(3, T_W)
    w = np.stack([rw.standard_normal((hidden, inter)) / np.sqrt(hidden) for _ in range(experts)])
    rd = rng_for(3, T_D)
    d = np.empty((rows, inter), dtype=np.float64)
    for e in range(experts):
        r0, r1 = offsets[e], offsets[e + 1]
        nu = 0.05 * rd.standard_normal(inter)
        d[r0:r1] = nu[None, :] + np.sqrt(1e-3) * rd.standard_normal((r1 - r0, inter))
    bf = torch.bfloat16
    return dict(x=_cast(x, bf), w=_cast(w, bf), d=_cast(d, bf), offsets=offsets)


def block_linear(name, l=16384):
    """One linear of the Qwen3-0.6B-like block sweep at l tokens."""
    k_in, n_out = QWEN3_06B_LINEARS[name]
    lid = list(QWEN3_06B_LINEARS).index(name)
    if name == "down":
        x = swiglu_activation(rng_for(4, T_X, lid), l, k_in)
    else:
        x = mean_biased_activation(rng_for(4, T_X, lid), l, k_in)
    w = weight(rng_for(4, T_W, lid), k_in, n_out)
    d = gradient(rng_for(4, T_D, lid), l, n_out)
    return dict(x=x, w=w, d=d)
