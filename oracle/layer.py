"""fp64 numpy oracle for one Qwen3-shaped attention layer (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may use this module.  It shares no code, table or helper with the HIP library.

The pages test the method on three Qwen3 sizes (1.7B, 4B, 8B) at contexts of
up to 128K (seventnews.com, "Empirical results that challenge the status
quo"), and one of them describes the method's cost as a few extra matrix products
per layer (news.ubos.tech, "How It Works in Practice"; a low-reliability page).
This module states the attention layer those models run, with the bifocal
attention in place of plain attention, so that its share of a layer can be
measured.  The layer is the Qwen3 attention block:

1. ``qkv = x W_qkv^T`` (no bias), split into Hq query heads, Hkv key heads and
   Hkv value heads of D = 128;
2. a per-head RMSNorm on the query and key heads (scale gamma_q, gamma_k;
   ``y = x / sqrt(mean(x^2) + eps) * gamma``);
3. RoPE at the tokens' original positions ``past + t`` (rotate-half pairs,
   theta_d = b^(-2d/D)): the keys and values are appended to the cache at those
   rows, keys rotated, values as they are;
4. attention of the new queries over the cache: bifocal (``oracle.bifocal``) or
   plain causal;
5. ``out = attn W_o^T`` (no bias).

Readings: the norm, the split order (all query heads, then key heads, then
value heads) and the absence of biases are those of the Qwen3 architecture the
pages evaluate; the pages themselves print none of it.

Parity pins (``tests/test_oracle_layer.py``): ``rms_norm_heads`` against torch's
fp64 ``rms_norm``, unit RMS and scale invariance; the whole layer at s <= L
against a torch fp64 composition (``linear``, ``rms_norm``, RoPE as complex
multiplication, ``scaled_dot_product_attention`` with GQA and a causal mask
offset by the past keys); at s > L against the per-pair brute force of
``oracle.bifocal`` on the normalised, unrotated heads; and a layer run in two
chunks against the same layer run at once.
"""

from __future__ import annotations

import numpy as np

from . import bifocal as _bf

__all__ = ["rms_norm_heads", "qwen3_attention_layer"]


def rms_norm_heads(x: np.ndarray, gamma: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis (one head of D values): x / sqrt(mean(x^2) + eps) * gamma."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def _split_heads(qkv: np.ndarray, hq: int, hkv: int, d: int):
    b, s, _ = qkv.shape
    q = qkv[..., :hq * d].reshape(b, s, hq, d)
    k = qkv[..., hq * d:(hq + hkv) * d].reshape(b, s, hkv, d)
    v = qkv[..., (hq + hkv) * d:].reshape(b, s, hkv, d)
    return q, k, v


def qwen3_attention_layer(x, w_qkv, gamma_q, gamma_k, w_o, n_q_heads, n_kv_heads, pretrained_window,
                          local_window, rope_base, past_k=None, past_v=None, eps=1e-6, bifocal=True,
                          schedule="grouped", return_heads=False, rows=None):
    """One attention layer over ``n_new`` new tokens appended to a cache.

    x        [B, n_new, H]                  hidden states of the new tokens
    w_qkv    [(Hq + 2 Hkv) D, H]            stacked q, k, v projections
    gamma_q, gamma_k [D]                    per-head RMSNorm scales
    w_o      [H, Hq D]                      output projection
    past_k, past_v [B, past, Hkv, D] or None: the cache before this call (keys
                                            rotated at their positions)

    Returns ``(out [B, n_new, H], k_cache, v_cache)`` with the caches of
    ``past + n_new`` rows; with ``return_heads`` also the normalised unrotated
    heads ``(q, k, v)`` and the attention output ``attn [B, n_new, Hq, D]``.
    Attention is ``oracle.bifocal.bifocal_three_pass`` under ``schedule`` (g from
    s = past + n_new) when ``bifocal``, else plain causal attention.  ``rows``
    selects new-token rows: ``out`` and ``attn`` then hold those rows only (the
    caches are always whole).
    """
    x = np.asarray(x, dtype=np.float64)
    b, n_new, _ = x.shape
    d = 128
    hq, hkv = int(n_q_heads), int(n_kv_heads)
    past = 0 if past_k is None else past_k.shape[1]
    qkv = x @ np.asarray(w_qkv, dtype=np.float64).T
    q, k, v = _split_heads(qkv, hq, hkv, d)
    q = rms_norm_heads(q, gamma_q, eps)
    k = rms_norm_heads(k, gamma_k, eps)
    theta = _bf.rope_frequencies(d, rope_base)
    pos = np.arange(past, past + n_new, dtype=np.float64)
    ang = (pos[:, None] * theta)[None, :, None, :]
    q_rot = _bf.rotate_half_pairs(q, ang)
    k_rot = _bf.rotate_half_pairs(k, ang)
    k_cache = k_rot if past_k is None else np.concatenate([np.asarray(past_k, np.float64), k_rot], axis=1)
    v_cache = v if past_v is None else np.concatenate([np.asarray(past_v, np.float64), v], axis=1)
    if bifocal:
        attn = _bf.bifocal_three_pass(q_rot, k_cache, v_cache, pretrained_window, local_window, rope_base,
                                      schedule=schedule, rows=rows)["out"]
    else:
        attn = _bf.plain_causal_attention(q_rot, k_cache, v_cache, rows=rows)[0]
    out = attn.reshape(b, attn.shape[1], hq * d) @ np.asarray(w_o, dtype=np.float64).T
    if return_heads:
        return out, k_cache, v_cache, (q, k, v), attn
    return out, k_cache, v_cache
