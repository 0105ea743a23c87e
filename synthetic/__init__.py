"""Seeded synthetic inputs shared by the GPU tests, the benchmark and the oracle.

This module draws random numbers and stores them as bf16; it holds none of
the quantization method's arithmetic.  bf16 conversion is done by torch
(round to nearest even).  There are no datasets or trained weights in this
project, so these tensors stand in for the pages' models: weight shapes of
the 1B / 2B / 3.9B Llama-style models the pages quantize (hidden 2048 with
2048x2048 and 2048<->5632 projections; 4096 and 11008 projections; 8192^2),
Gaussian or Student-t weights at sigma 0.02 and N(0, 1) activations.

Two generators with the same recipe:

* host: ``numpy.random.Generator(PCG64(seed))`` in float64 -> float32 ->
  bf16.  Used wherever the oracle must see the whole input.
* device: ``torch.Generator('cuda')`` (Philox) in float32 -> bf16.  Used for
  the full-size stacks (up to 1.2 G weights) where host generation would take
  minutes; the oracle then gets the sampled rows copied back to the host.

Seeds: ``seed(c, i, role) = 1000*c + 2*i + role`` (role 0 = weight, 1 =
activation), except the single 2048x2048 case whose weight uses seed 0 and
activation seed 1.
"""

import numpy as np
import torch


def seed(config, index, role):
    if config == 1:
        return role
    return 1000 * config + 2 * index + role


def _to_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _rng(s):
    return np.random.Generator(np.random.PCG64(s))


# ---------------------------------------------------------------- host (numpy)
def normal_bf16(shape, sigma, s):
    return _to_bf16_bits(_rng(s).standard_normal(shape) * sigma)


def student_t_bf16(shape, nu, sigma, s):
    """Student-t with nu degrees of freedom scaled to standard deviation sigma."""
    scale = sigma * np.sqrt((nu - 2.0) / nu)
    return _to_bf16_bits(_rng(s).standard_t(nu, size=shape) * scale)


def normal_outliers_bf16(shape, sigma, p, value, s):
    """N(0, sigma^2) where each element is replaced with probability p by +-value."""
    g = _rng(s)
    w = g.standard_normal(shape) * sigma
    hit = g.random(shape) < p
    sgn = np.where(g.random(shape) < 0.5, -1.0, 1.0)
    return _to_bf16_bits(np.where(hit, sgn * value, w))


# ---------------------------------------------------------------- device (torch)
def _gen(s, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(s))
    return g


def normal_bf16_device(shape, sigma, s, device="cuda"):
    g = _gen(s, device)
    return (torch.randn(shape, generator=g, device=device) * sigma).to(torch.bfloat16)


def student_t_bf16_device(shape, nu, sigma, s, device="cuda"):
    """t = z / sqrt(chi2_nu / nu) with chi2_nu a sum of nu squared normals."""
    g = _gen(s, device)
    z = torch.randn(shape, generator=g, device=device)
    chi = torch.zeros(shape, device=device)
    for _ in range(int(nu)):
        chi += torch.randn(shape, generator=g, device=device) ** 2
    t = z / torch.sqrt(chi / nu)
    return (t * (sigma * float(np.sqrt((nu - 2.0) / nu)))).to(torch.bfloat16)


def normal_outliers_bf16_device(shape, sigma, p, value, s, device="cuda"):
    g = _gen(s, device)
    w = torch.randn(shape, generator=g, device=device) * sigma
    hit = torch.rand(shape, generator=g, device=device) < p
    sgn = torch.where(torch.rand(shape, generator=g, device=device) < 0.5, -1.0, 1.0)
    return torch.where(hit, sgn * value, w).to(torch.bfloat16)


# ---------------------------------------------------------------- workloads
def llama1b_stack_shapes(blocks=24, hidden=2048, ffn=5632):
    """The 1B decode stack: per block q, k, v, o [h, h]; gate, up [f, h]; down [h, f]
    (shapes [out_features N, in_features K]), in block order."""
    per_block = [(hidden, hidden)] * 4 + [(ffn, hidden)] * 2 + [(hidden, ffn)]
    return per_block * blocks


def llama39b_shapes():
    """One of each 3.9B-sized projection: [4096, 4096], [11008, 4096], [4096, 11008]."""
    return [(4096, 4096), (11008, 4096), (4096, 11008)]


def minicpm2b_shapes(layers=32, per_layer=7, hidden=2048):
    """The 2B model's 224 square 2048x2048 matrices (32 layers x 7)."""
    return [(hidden, hidden)] * (layers * per_layer)
