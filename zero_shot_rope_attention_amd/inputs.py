"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it draws N(0, 1) samples with a
seeded numpy generator and rounds them to bfloat16 (round to nearest even),
returning the raw bf16 bit patterns.  Both the HIP path (as device bf16
tensors) and the fp64 oracle (as exact fp64 values of those bf16 numbers) are
fed from the same bits.

Recipe: ``numpy.random.default_rng([workload_id, tensor_id])`` with tensor_id
0/1/2 for Q/K/V, ``standard_normal(shape, float32)`` -> bf16 RNE.  The vectors
are taken *as* the cached, already position-rotated Q and K (rotating an
isotropic Gaussian leaves its distribution unchanged).

The attention layer's inputs (``make_layer``) use tensor ids 3..7: hidden states
x ~ N(0, 1); projections with N(0, 1/fan_in) entries, so that the projected heads
have unit variance; RMSNorm scales 1 + N(0, 1/16).
"""

from __future__ import annotations

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2
TENSOR_X, TENSOR_WQKV, TENSOR_WO, TENSOR_GQ, TENSOR_GK = 3, 4, 5, 6, 7


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.
    NaNs are not expected in these inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_bf16(workload_id: int, tensor_id: int, shape, scale: float = 1.0,
                chunk: int = 1 << 24) -> np.ndarray:
    """Seeded N(0, scale^2) samples rounded to bf16, as uint16 bits of ``shape``.
    Generated in chunks so that large tensors never hold a full float32 copy."""
    rng = np.random.default_rng([int(workload_id), int(tensor_id)])
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        x = rng.standard_normal(m, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[i:i + m] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def make_qkv(workload_id: int, batch: int, n_q: int, n_kv: int, n_q_heads: int,
             n_kv_heads: int, head_dim: int, q_scale: float = 1.0):
    """Q [B, n_q, Hq, D], K and V [B, n_kv, Hkv, D], as bf16 bit arrays."""
    q = normal_bf16(workload_id, TENSOR_Q, (batch, n_q, n_q_heads, head_dim), q_scale)
    k = normal_bf16(workload_id, TENSOR_K, (batch, n_kv, n_kv_heads, head_dim))
    v = normal_bf16(workload_id, TENSOR_V, (batch, n_kv, n_kv_heads, head_dim))
    return q, k, v


def make_layer(workload_id: int, batch: int, n_new: int, hidden: int, n_q_heads: int, n_kv_heads: int,
               head_dim: int = 128):
    """Inputs of one attention layer as bf16 bit arrays: x [B, n_new, hidden],
    w_qkv [(Hq + 2 Hkv) D, hidden], w_o [hidden, Hq D], gamma_q and gamma_k [D]."""
    x = normal_bf16(workload_id, TENSOR_X, (batch, n_new, hidden))
    w_qkv = normal_bf16(workload_id, TENSOR_WQKV, ((n_q_heads + 2 * n_kv_heads) * head_dim, hidden),
                        1.0 / np.sqrt(hidden))
    w_o = normal_bf16(workload_id, TENSOR_WO, (hidden, n_q_heads * head_dim), 1.0 / np.sqrt(n_q_heads * head_dim))
    gammas = []
    for tid in (TENSOR_GQ, TENSOR_GK):
        z = np.random.default_rng([int(workload_id), tid]).standard_normal(head_dim, dtype=np.float32)
        gammas.append(f32_to_bf16_bits(np.float32(1.0) + np.float32(0.25) * z))
    return x, w_qkv, w_o, gammas[0], gammas[1]
