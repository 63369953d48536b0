"""Seeded synthetic inputs for the NVFP4 quantize -> GEMM path.

This module holds input generation only -- none of the method's arithmetic.
Both the GPU path and the CPU oracle are fed from here, as bf16 bit patterns
(numpy uint16), so that they see identical inputs.

Distributions stand in for the 12B-model layer data the pages talk about
("Pretraining Large Language Models with NVFP4", Technische Zusammenfassung
section 4: a 12B hybrid Mamba-Transformer); no dataset or trained weights are
used.  Recipe (all draws float64 from numpy.random.default_rng(seed), cast to
fp32, then to bf16 with round-to-nearest-even):

  activations, small : N(0, 1); 0.1 % of entries (positions drawn without
                       replacement) multiplied by 50 as outliers
  activations        : Student-t(df=4) scaled to unit variance (x sqrt(1/2))
  activations, heavy : Student-t(df=3) scaled to unit variance (x sqrt(1/3))
  weights            : N(0, 0.02)
  gradients          : 1e-3 * exp(2 z_row) * g, z_row ~ N(0,1) per row,
                       g ~ N(0,1) per element (log-normal row magnitudes,
                       sigma = 2), which puts some rows' block scales into the
                       E4M3 subnormal and zero range.

The 4-block MLP training step (tokens 16384 = batch 4 x sequence 4096, hidden
5120, FFN 20480; blocks of an up- and a down-projection; the last block kept
in BF16) draws its much larger inputs on the GPU with torch's seeded
generator instead, same distributions, activations Student-t(3):
  Student-t(df), integer df : Z / sqrt((Z_1^2 + ... + Z_df^2) / df), all
                              standard normals, scaled to unit variance
Each linear layer gets its own inputs (layer seed = seed + 4096 * index);
the activations of one layer are not the output of the previous one.
"""
from dataclasses import dataclass

import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round-to-nearest-even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(u) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(rng, shape, std):
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def normal_with_outliers(rng, shape, frac=1e-3, factor=50.0):
    x = rng.standard_normal(shape)
    n = int(round(frac * x.size))
    pos = rng.choice(x.size, size=n, replace=False)
    x.reshape(-1)[pos] *= factor
    return f32_to_bf16_bits(x.astype(np.float32))


def student_t_unit_var(rng, shape, df):
    x = rng.standard_t(df, size=shape) * np.sqrt((df - 2.0) / df)
    return f32_to_bf16_bits(x.astype(np.float32))


def lognormal_rows(rng, shape, base=1e-3, sigma=2.0):
    rows, cols = shape
    z = rng.standard_normal((rows, 1))
    g = rng.standard_normal(shape)
    return f32_to_bf16_bits((base * np.exp(sigma * z) * g).astype(np.float32))


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

@dataclass
class LayerShapes:
    M: int   # tokens
    K: int   # layer input features
    N: int   # layer output features


SMALL = LayerShapes(256, 256, 256)
LAYER_12B = LayerShapes(8192, 5120, 20480)     # 12B-style MLP up-projection
STEP_12B_M = 16384                              # batch 4 x seq 4096


def small_fprop(seed=0):
    """256^3 fprop: X ~ N(0,1) with 0.1 % x50 outliers, W ~ N(0, 0.02)."""
    rng = np.random.default_rng(seed)
    X = normal_with_outliers(rng, (SMALL.M, SMALL.K))
    W = normal(rng, (SMALL.N, SMALL.K), 0.02)
    return X, W


def layer_inputs(shapes: LayerShapes, seed=0, act_df=4, with_x=True, with_w=True, with_dy=True):
    """X (M x K, Student-t), W (N x K, N(0, 0.02)), dY (M x N, log-normal rows).

    Drawn in the order X, W, dY from one generator.
    """
    rng = np.random.default_rng(seed)
    out = {}
    if with_x:
        out["X"] = student_t_unit_var(rng, (shapes.M, shapes.K), act_df)
    if with_w:
        out["W"] = normal(rng, (shapes.N, shapes.K), 0.02)
    if with_dy:
        out["dY"] = lognormal_rows(rng, (shapes.M, shapes.N))
    return out


MLP_TOKENS = 16384
MLP_HIDDEN = 5120
MLP_FFN = 20480
MLP_BLOCKS = 4
MLP_SEED = 1


def mlp_layers(tokens=MLP_TOKENS, hidden=MLP_HIDDEN, ffn=MLP_FFN, blocks=MLP_BLOCKS):
    """Shapes of the linear layers of the MLP stack, in order: per block an
    up-projection (hidden -> ffn) and a down-projection (ffn -> hidden)."""
    out = []
    for _ in range(blocks):
        out.append(LayerShapes(tokens, hidden, ffn))
        out.append(LayerShapes(tokens, ffn, hidden))
    return out


def layer_seed(base_seed: int, index: int) -> int:
    return base_seed + 4096 * index


def layer_inputs_device(torch, device, shapes: LayerShapes, seed, act_df=3):
    """X (M x K, Student-t(act_df) at unit variance), W (N x K, N(0, 0.02)) and
    dY (M x N, log-normal row magnitudes) as bf16 tensors on `device`, drawn
    in that order from torch's generator seeded with `seed`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def randn(shape):
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)

    M, K, N = shapes.M, shapes.K, shapes.N
    z = randn((M, K))
    chi2 = torch.zeros_like(z)
    for _ in range(act_df):
        e = randn((M, K))
        chi2.addcmul_(e, e)
        del e
    x = (z / torch.sqrt(chi2 / act_df)) * ((act_df - 2.0) / act_df) ** 0.5
    del z, chi2
    out = {"X": x.to(torch.bfloat16)}
    del x
    out["W"] = (randn((N, K)) * 0.02).to(torch.bfloat16)
    row = torch.exp(2.0 * randn((M, 1))) * 1e-3
    out["dY"] = (row * randn((M, N))).to(torch.bfloat16)
    return out


def sr_seed(base_seed: int, k: int) -> int:
    """Seed of the k-th stochastic-rounding call of a workload."""
    return base_seed + 100 + k


def rht_seed(base_seed: int) -> int:
    """Seed from which the RHT sign vector of a workload is drawn."""
    return base_seed + 1000
