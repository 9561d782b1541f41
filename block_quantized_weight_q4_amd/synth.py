"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no arithmetic of the method: it never decodes a block, never
forms a weight and never takes a product.  It only writes random bytes and
fp16 / int8 fields at their offsets inside each block.

Block fields written here (byte offsets inside one block):

* Q4_0 (18 B): fp16 ``d`` at 0, 16 quant bytes at 2.
* Q4_K (144 B): fp16 ``d`` at 0, fp16 ``dmin`` at 2, 12 scale bytes at 4,
  128 quant bytes at 16.
* Q6_K (210 B): 128 low-bit bytes at 0, 64 high-bit bytes at 128, 16 int8
  scales at 192, fp16 ``d`` at 208.
* Q5_K (176 B): fp16 ``d`` at 0, fp16 ``dmin`` at 2, 12 scale bytes at 4,
  32 fifth-bit bytes at 16, 128 quant bytes at 48.

Uniform quants and uniform 6-bit (scale, min) pairs are produced by uniform
random *bytes*: every bit of the quant bytes and of Q4_K's 12 scale bytes
belongs to exactly one field, so uniform bytes give independent, uniform
fields (4-bit quants 0..15, 6-bit quants 0..63, 6-bit scales/mins 0..63)
without this module knowing how the bits are arranged.

Seeds: ``seed = 0x67510000 + workload number``; each tensor draws from its own
numpy PCG64 stream ``default_rng([seed, tensor_index])``.
"""
from __future__ import annotations

import numpy as np

BLOCK = {"q4_0": (32, 18), "q4_k": (256, 144), "q6_k": (256, 210), "q5_k": (256, 176)}
SEED_BASE = 0x67510000


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def _f16_bytes(vals: np.ndarray) -> np.ndarray:
    """fp16 (round to nearest even, numpy's cast) as little-endian byte pairs."""
    return np.asarray(vals, np.float64).astype(np.float16).view(np.uint8).reshape(-1, 2)


def blocks_q4_0(g: np.random.Generator, n_blocks: int, d_scale: float = 0.01) -> np.ndarray:
    """d = fp16(|N(0,1)| * d_scale); quants uniform 0..15."""
    out = np.empty((n_blocks, 18), np.uint8)
    out[:, 0:2] = _f16_bytes(np.abs(g.standard_normal(n_blocks)) * d_scale)
    out[:, 2:18] = g.integers(0, 256, size=(n_blocks, 16), dtype=np.uint8)
    return out


def blocks_q4_k(g: np.random.Generator, n_blocks: int, d_scale: float = 1e-3) -> np.ndarray:
    """d, dmin = fp16(|N(0,1)| * d_scale); scales/mins uniform 0..63; quants 0..15."""
    out = np.empty((n_blocks, 144), np.uint8)
    out[:, 0:2] = _f16_bytes(np.abs(g.standard_normal(n_blocks)) * d_scale)
    out[:, 2:4] = _f16_bytes(np.abs(g.standard_normal(n_blocks)) * d_scale)
    out[:, 4:16] = g.integers(0, 256, size=(n_blocks, 12), dtype=np.uint8)
    out[:, 16:144] = g.integers(0, 256, size=(n_blocks, 128), dtype=np.uint8)
    return out


def blocks_q6_k(g: np.random.Generator, n_blocks: int, d_scale: float = 1e-3,
                sc_sigma: float = 16.0) -> np.ndarray:
    """6-bit quants uniform 0..63; int8 scales = clip(rint(N(0, sc_sigma)), +-127);
    d = fp16(|N(0,1)| * d_scale)."""
    out = np.empty((n_blocks, 210), np.uint8)
    out[:, 0:192] = g.integers(0, 256, size=(n_blocks, 192), dtype=np.uint8)
    sc = np.clip(np.rint(g.standard_normal((n_blocks, 16)) * sc_sigma), -127, 127).astype(np.int8)
    out[:, 192:208] = sc.view(np.uint8)
    out[:, 208:210] = _f16_bytes(np.abs(g.standard_normal(n_blocks)) * d_scale)
    return out


def blocks_q5_k(g: np.random.Generator, n_blocks: int, d_scale: float = 1e-3) -> np.ndarray:
    """d, dmin = fp16(|N(0,1)| * d_scale); scales/mins uniform 0..63; 5-bit
    quants uniform 0..31 (uniform quant and fifth-bit bytes)."""
    out = np.empty((n_blocks, 176), np.uint8)
    out[:, 0:2] = _f16_bytes(np.abs(g.standard_normal(n_blocks)) * d_scale)
    out[:, 2:4] = _f16_bytes(np.abs(g.standard_normal(n_blocks)) * d_scale)
    out[:, 4:176] = g.integers(0, 256, size=(n_blocks, 172), dtype=np.uint8)
    return out


def blocks(t: str, g: np.random.Generator, n_blocks: int) -> np.ndarray:
    return {"q4_0": blocks_q4_0, "q4_k": blocks_q4_k, "q6_k": blocks_q6_k, "q5_k": blocks_q5_k}[t](g, n_blocks)


def weight(t: str, g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """Packed [N][K/elems blocks] matrix as uint8 [N, row_bytes] (rows back to back)."""
    elems, nbytes = BLOCK[t]
    assert K % elems == 0
    return blocks(t, g, N * (K // elems)).reshape(N, (K // elems) * nbytes)


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(shape).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (no NaN inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact expansion of bf16 bit patterns to fp32."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def router_logits(g: np.random.Generator, n_tokens: int, n_experts: int) -> np.ndarray:
    """Seeded router scores: N(0,1) logits [n_tokens][n_experts], fp32."""
    return g.standard_normal((n_tokens, n_experts)).astype(np.float32)
