"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

Holds none of the method's arithmetic: it only draws random tensors with the
shapes and value distributions of the workloads (LLaMA-7B / 65B-class layer
shapes, weights ~ N(0, sigma) or a scaled Student-t, activations ~ N(0, 1)).
Every host tensor is drawn in float64 with NumPy's PCG64 seeded by
(seed, *key), scaled, then rounded float64 -> float32 -> bfloat16 (round to
nearest even, done by PyTorch's dtype conversion). The same bfloat16 bits are
then handed to the HIP library and to the oracle.
"""

import numpy as np
import torch


def _rng(seed, key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, key)])))


def to_bf16(x64):
    """float64 array -> (bf16 torch CPU tensor, float32 numpy array of the same values)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64).astype(np.float32)).to(torch.bfloat16)
    return t, t.to(torch.float32).numpy()


def normal(shape, std=1.0, seed=0, key=(0,)):
    """N(0, std^2) as bfloat16: (torch CPU bf16, numpy float32 values)."""
    g = _rng(seed, key)
    return to_bf16(g.standard_normal(shape) * std)


def student_t(shape, df=5.0, scale=0.02, seed=0, key=(0,)):
    """scale * Student-t(df) as bfloat16 (heavy tails: stresses block absmax)."""
    g = _rng(seed, key)
    return to_bf16(g.standard_t(df, size=shape) * scale)


def device_normal_bf16(n, std, seed, device):
    """N(0, std^2) bf16 drawn on the device (for stacks too large for the host)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    step = 1 << 28
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = (torch.randn(e - s, generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)
    return out


# Tensor ids used in keys: (config, layer, tensor_id)
W_ID, A_ID, B_ID, X_ID, DY_ID = 0, 1, 2, 3, 4


def linear_case(M, N, K, r, seed=0, cfg=0, layer=0, w_std=0.02, ab_std=0.02, w_dist="normal"):
    """Inputs of one LoRA linear: dict of (torch bf16 CPU, numpy float32) pairs."""
    if w_dist == "student_t":
        W = student_t((N, K), 5.0, w_std, seed, (cfg, layer, W_ID))
    else:
        W = normal((N, K), w_std, seed, (cfg, layer, W_ID))
    return {
        "W": W,
        "A": normal((r, K), ab_std, seed, (cfg, layer, A_ID)),
        "B": normal((N, r), ab_std, seed, (cfg, layer, B_ID)),
        "X": normal((M, K), 1.0, seed, (cfg, layer, X_ID)),
        "dY": normal((M, N), 1.0, seed, (cfg, layer, DY_ID)),
    }


# The seven projections of a LLaMA decoder layer: (name, out N, in K).
def llama_linears(hidden, ffn):
    return [("q", hidden, hidden), ("k", hidden, hidden), ("v", hidden, hidden), ("o", hidden, hidden),
            ("gate", ffn, hidden), ("up", ffn, hidden), ("down", hidden, ffn)]
