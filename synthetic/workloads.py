"""Seeded input generators for the five quantization workloads.

Each generator draws float32 values with numpy's PCG64 ``default_rng(seed)`` and rounds them to
BF16 with round-to-nearest-even (torch CPU ``.to(torch.bfloat16)``). BF16 tensors are returned as
``numpy.uint16`` arrays of raw bit patterns, row-major. Every generator takes an optional shape so
that tests can draw small tensors with the same value distribution.

Value structure follows the pages' discussion of LLM tensors: Gaussian activations with
injected outliers, token-wise heavy tails, and gradients with a wide dynamic range.
"""
import numpy as np
import torch

__all__ = [
    "bf16_bits", "bf16_to_f32", "inject_outliers",
    "SHAPES", "small_tensor", "per_tensor_small", "per_tensor_activation", "delayed_base",
    "delayed_sigmas", "delayed_step_input", "mx_gradient", "block_weight", "token_activation",
]

SHAPES = {
    "per_tensor_small": (256, 512),
    "per_tensor_activation": (8192, 8192),
    "delayed": (4096, 14336),
    "mx_gradient": (16384, 4096),
    "block_weight": (7168, 18432),
    "token_activation": (8192, 7168),
}


def bf16_bits(f32):
    """float32 array -> uint16 BF16 bit patterns (round to nearest, ties to even)."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_to_f32(bits):
    """uint16 BF16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def inject_outliers(rng, x, frac, factor):
    """Multiply round(frac * x.size) distinct entries, chosen uniformly, by factor (in place)."""
    flat = x.reshape(-1)
    k = int(round(frac * flat.size))
    if k > 0:
        idx = rng.choice(flat.size, size=k, replace=False)
        flat[idx] *= np.float32(factor)
    return x


def small_tensor(rows, cols, seed=0, scale=1.0):
    """Plain N(0, scale^2) BF16 tensor."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(scale))


def per_tensor_small(rows=256, cols=512, seed=1):
    """256x512 N(0,1) with 0.5% of the entries scaled by 200."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    return bf16_bits(inject_outliers(rng, x, 0.005, 200.0))


def per_tensor_activation(rows=8192, cols=8192, seed=2):
    """Activation N(0,1) with 0.1% of the entries scaled by 1000."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    return bf16_bits(inject_outliers(rng, x, 0.001, 1000.0))


def delayed_base(rows=4096, cols=14336, seed=3):
    """Fixed float32 N(0,1) base tensor Z of the drifting-std sequence."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, cols), dtype=np.float32)


def delayed_sigmas(steps=100, seed=30):
    """Per-step std sigma_t = 0.5 * 8^u_t, u_t ~ U[0,1) i.i.d., i.e. log-uniform in [0.5, 4)."""
    rng = np.random.default_rng(seed)
    u = rng.random(steps)
    return (0.5 * np.power(8.0, u)).astype(np.float32)


def delayed_step_input(z, sigma):
    """X_t = bf16(fl32(sigma_t * Z))."""
    return bf16_bits(z * np.float32(sigma))


def mx_gradient(rows=16384, cols=4096, seed=4):
    """Gradient-like tensor: Laplace(0, b=1e-3) with 0.01% of the entries scaled by 1e4."""
    rng = np.random.default_rng(seed)
    x = rng.laplace(0.0, 1e-3, size=(rows, cols)).astype(np.float32)
    return bf16_bits(inject_outliers(rng, x, 1e-4, 1e4))


def block_weight(rows=7168, cols=18432, seed=51):
    """Weight N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02))


def token_activation(rows=8192, cols=7168, seed=52):
    """Token-wise heavy tails: x[t, :] = |T_t| * z[t, :], T_t ~ Student-t(3), z ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    t = np.abs(rng.standard_t(3.0, size=(rows, 1))).astype(np.float32)
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    return bf16_bits(z * t)
