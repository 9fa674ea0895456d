"""Seeded synthetic inputs shaped like CogVideoX linear-layer activations.

This module only draws random numbers and rounds them to bf16; it holds none
of the method's arithmetic, and both the GPU path's tests/benchmark and the
CPU oracle's checks take their inputs from it.  The 6Bit-Diffusion pages
measure on CogVideoX-2B/5B (summary, section four); neither the models nor
their evaluation suites are available, so these generators stand in for the
activations at the hidden sizes and token count of those models:
M = 17776 tokens = 13 latent frames x 1350 patches + 226 text tokens,
hidden 1920 (2B) or 3072 (5B), FFN inner 12288 (5B).

Host tensors are numpy uint16 arrays of bf16 bit patterns; float32 values
are rounded to bf16 by torch (round to nearest even).
"""
import math

import numpy as np
import torch

M_COGVIDEOX = 13 * 1350 + 226  # 17776


def rng_for(cfg, tensor_id, seed=0):
    """numpy PCG64 generator for (seed, config, tensor)."""
    return np.random.default_rng(np.random.SeedSequence([seed, cfg, tensor_id]))


def to_bf16_bits(x):
    """float32 numpy -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(x16):
    return (np.ascontiguousarray(x16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(K, frac, rng):
    """round(frac * K) channel indices drawn by a seeded permutation."""
    n = int(round(frac * K))
    return np.sort(rng.permutation(K)[:n])


def gaussian_outliers(M, K, frac, factor, rng, chunk=2048):
    """N(0, 1) entries with round(frac*K) channels scaled by `factor`."""
    ch = outlier_channels(K, frac, rng)
    out = np.empty((M, K), np.uint16)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        z = rng.standard_normal((r1 - r0, K), dtype=np.float32)
        z[:, ch] *= np.float32(factor)
        out[r0:r1] = to_bf16_bits(z)
    return out


def lognormal_tokens(M, K, rng, sigma=0.5, chunk=2048):
    """x[m, k] = g_m * z_mk with z ~ N(0, 1), g_m ~ LogNormal(0, sigma)."""
    g = rng.lognormal(0.0, sigma, size=M).astype(np.float32)
    out = np.empty((M, K), np.uint16)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        z = rng.standard_normal((r1 - r0, K), dtype=np.float32)
        out[r0:r1] = to_bf16_bits(z * g[r0:r1, None])
    return out


def smooth_video_tokens(F, H, W, K, rng, outlier_frac=0.01, factor=20.0, noise=0.05):
    """Video tokens of an F x H x W grid (frame outermost) whose values vary
    slowly in space and time: per channel a base value (1% of channels x20),
    linear ramps over frames, rows and columns, and a little independent
    noise.  bf16 bits [F * H * W, K]."""
    base = rng.standard_normal(K).astype(np.float32)
    base[outlier_channels(K, outlier_frac, rng)] *= np.float32(factor)
    ramps = rng.standard_normal((3, K)).astype(np.float32) * np.float32(0.3)
    f = np.arange(F, dtype=np.float32)[:, None, None, None] / np.float32(max(F, 1))
    h = np.arange(H, dtype=np.float32)[None, :, None, None] / np.float32(max(H, 1))
    w = np.arange(W, dtype=np.float32)[None, None, :, None] / np.float32(max(W, 1))
    x = base + f * ramps[0] + h * ramps[1] + w * ramps[2]
    x = x + rng.standard_normal((F, H, W, K)).astype(np.float32) * np.float32(noise)
    return to_bf16_bits(x.reshape(F * H * W, K))


def gelu_student_t(M, K, rng, nu=3.0, chunk=1024):
    """GELU (exact erf form) of N(0, 1) plus unit-scale Student-t(nu) noise:
    the input of an FFN down-projection with heavy tails."""
    from scipy.special import erf
    out = np.empty((M, K), np.uint16)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        z = rng.standard_normal((r1 - r0, K))
        t = rng.standard_t(nu, size=(r1 - r0, K))
        x = 0.5 * z * (1.0 + erf(z / math.sqrt(2.0))) + t
        out[r0:r1] = to_bf16_bits(x.astype(np.float32))
    return out


def gaussian(M, K, std, rng, chunk=4096):
    """N(0, std) entries (std is the standard deviation)."""
    out = np.empty((M, K), np.uint16)
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        z = rng.standard_normal((r1 - r0, K), dtype=np.float32) * np.float32(std)
        out[r0:r1] = to_bf16_bits(z)
    return out


# The single-layer workloads.  Each entry: activation generator, weight shape
# and the path(s) run on it.
CONFIGS = {
    1: dict(name="single linear 1024x1024x1024, 1% outlier channels x20",
            M=1024, K=1024, N=1024, had_block=64, paths=("nvfp4", "int8"), out="f32"),
    2: dict(name="CogVideoX-2B QKV projection 1920->5760, INT8",
            M=M_COGVIDEOX, K=1920, N=5760, had_block=128, paths=("int8",), out="bf16"),
    3: dict(name="CogVideoX-5B FFN up-projection 3072->12288, NVFP4",
            M=M_COGVIDEOX, K=3072, N=12288, had_block=128, paths=("nvfp4",), out="bf16"),
    4: dict(name="CogVideoX-5B FFN down-projection 12288->3072, INT8",
            M=M_COGVIDEOX, K=12288, N=3072, had_block=128, paths=("int8",), out="bf16"),
}


def config_activations(cfg, M=None, seed=0):
    """Activations of a single-layer config (optionally only the first M
    rows' worth of shape, drawn from the same recipe)."""
    c = CONFIGS[cfg]
    M = c["M"] if M is None else M
    K = c["K"]
    rng = rng_for(cfg, 0, seed)
    if cfg == 1:
        return gaussian_outliers(M, K, 0.01, 20.0, rng)
    if cfg == 2:
        return gaussian_outliers(M, K, 0.005, 30.0, rng)
    if cfg == 3:
        return lognormal_tokens(M, K, rng)
    if cfg == 4:
        return gelu_student_t(M, K, rng)
    raise ValueError(cfg)


def config_weights(cfg, seed=0):
    """bf16 weights [N, K] ~ N(0, 0.02) of a single-layer config."""
    c = CONFIGS[cfg]
    return gaussian(c["N"], c["K"], 0.02, rng_for(cfg, 1, seed))


# ------------------------------------------------------------------ schedule
# The dynamic schedule: CogVideoX-5B blocks, four linears each, over
# denoising steps.  Per (block, layer, step) the previous step's module
# output is the layer input plus N(0, s) noise, s ~ U(0.01, 0.3).

SCHEDULE_LAYERS = (("qkv", 3072, 9216), ("out", 3072, 3072),
                   ("ffn_up", 3072, 12288), ("ffn_down", 12288, 3072))


def schedule_noise_levels(blocks, steps, seed=0):
    """s[block, layer, step] ~ U(0.01, 0.3) from a seeded host generator."""
    rng = rng_for(5, 0, seed)
    return rng.uniform(0.01, 0.3, size=(blocks, len(SCHEDULE_LAYERS), steps))


def device_gaussian(shape, std, generator, device, dtype=torch.bfloat16):
    """N(0, std) drawn on the device with a seeded torch generator."""
    x = torch.randn(shape, generator=generator, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def device_noisy_copy(x, s, generator):
    """x + N(0, s), computed in float32 and rounded to bf16 (the previous
    step's module output in the schedule)."""
    n = torch.randn(x.shape, generator=generator, device=x.device, dtype=torch.float32)
    return (x.float() + n.mul_(s)).to(torch.bfloat16)
