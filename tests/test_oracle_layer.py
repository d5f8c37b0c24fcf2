"""Pins for the Qwen3-shaped attention layer of the oracle (CPU only).

The layer (oracle.layer) chains library-free fp64 steps: projection, per-head
RMSNorm, RoPE at the tokens' positions, bifocal or plain attention over the
cache, output projection.  It is checked against an independent torch fp64
composition of library routines where the method is the base model (s <= L),
against the per-pair brute force of the bifocal oracle beyond L, and against
itself run in two chunks.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import layer as ol

D = 128


def _weights(seed, hidden, hq, hkv):
    rng = np.random.default_rng(seed)
    w_qkv = rng.standard_normal(((hq + 2 * hkv) * D, hidden)) / math.sqrt(hidden)
    w_o = rng.standard_normal((hidden, hq * D)) / math.sqrt(hq * D)
    gq = rng.uniform(0.5, 1.5, D)
    gk = rng.uniform(0.5, 1.5, D)
    return w_qkv, gq, gk, w_o


def _torch_layer(x, w_qkv, gq, gk, w_o, hq, hkv, base, past_k=None, past_v=None, eps=1e-6):
    # library routines only: linear, rms_norm, complex multiplication, SDPA with GQA
    xt = torch.from_numpy(x)
    b, n, _ = x.shape
    past = 0 if past_k is None else past_k.shape[1]
    qkv = F.linear(xt, torch.from_numpy(w_qkv))
    q, k, v = torch.split(qkv, [hq * D, hkv * D, hkv * D], dim=-1)
    q = F.rms_norm(q.reshape(b, n, hq, D), (D,), weight=torch.from_numpy(gq), eps=eps)
    k = F.rms_norm(k.reshape(b, n, hkv, D), (D,), weight=torch.from_numpy(gk), eps=eps)
    v = v.reshape(b, n, hkv, D)
    inv = base ** (-torch.arange(0, D // 2, dtype=torch.float64) * 2.0 / D)
    pos = torch.arange(past, past + n, dtype=torch.float64)
    turn = torch.polar(torch.ones(n, D // 2, dtype=torch.float64), pos[:, None] * inv[None, :])[None, :, None, :]

    def rope(t):
        z = torch.complex(t[..., :D // 2], t[..., D // 2:]) * turn
        return torch.cat([z.real, z.imag], dim=-1)

    q, k = rope(q), rope(k)
    if past_k is not None:
        k = torch.cat([torch.from_numpy(past_k), k], dim=1)
        v = torch.cat([torch.from_numpy(past_v), v], dim=1)
    s = past + n
    mask = torch.arange(s)[None, :] <= (past + torch.arange(n))[:, None]
    attn = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), attn_mask=mask,
                                          enable_gqa=True).transpose(1, 2)
    return F.linear(attn.reshape(b, n, hq * D), torch.from_numpy(w_o)).numpy()


def test_rms_norm_heads_pins():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 5, 3, D)) * 3.0
    g = rng.uniform(0.5, 2.0, D)
    y = ol.rms_norm_heads(x, g, 1e-6)
    ref = F.rms_norm(torch.from_numpy(x), (D,), weight=torch.from_numpy(g), eps=1e-6).numpy()
    assert np.abs(y - ref).max() <= 1e-13
    y1 = ol.rms_norm_heads(x, np.ones(D), 0.0)
    assert np.allclose(np.sqrt(np.mean(y1 * y1, axis=-1)), 1.0, atol=1e-13)     # unit RMS
    assert np.abs(ol.rms_norm_heads(7.5 * x, g, 0.0) - ol.rms_norm_heads(x, g, 0.0)).max() <= 1e-13


@pytest.mark.parametrize("b,n,hidden,hq,hkv,past", [(1, 40, 64, 2, 1, 0), (2, 17, 96, 4, 2, 0), (1, 9, 64, 4, 1, 23)])
def test_layer_within_window_matches_torch(b, n, hidden, hq, hkv, past):
    w_qkv, gq, gk, w_o = _weights(10 + n, hidden, hq, hkv)
    rng = np.random.default_rng(20 + n)
    x = rng.standard_normal((b, n, hidden))
    pk = pv = None
    if past:
        xp = rng.standard_normal((b, past, hidden))
        _, pk, pv = ol.qwen3_attention_layer(xp, w_qkv, gq, gk, w_o, hq, hkv, 1024, 16, 1e4)
    # s <= L: the bifocal layer is the base model; so is the plain one
    for bif in (True, False):
        out, kc, vc = ol.qwen3_attention_layer(x, w_qkv, gq, gk, w_o, hq, hkv, 1024, 16, 1e4, pk, pv, bifocal=bif)
        ref = _torch_layer(x, w_qkv, gq, gk, w_o, hq, hkv, 1e4, pk, pv)
        assert np.abs(out - ref).max() <= 1e-12
        assert kc.shape == (b, past + n, hkv, D) and vc.shape == kc.shape


@pytest.mark.parametrize("schedule", list(oracle.SCHEDULES))
def test_layer_beyond_window_matches_bruteforce(schedule):
    # s = 70 > L = 16: the attention step is the per-pair brute force on the
    # normalised, unrotated heads (positions 0..69)
    b, n, hidden, hq, hkv, big_l, w, base = 1, 70, 64, 4, 2, 16, 5, 1e4
    w_qkv, gq, gk, w_o = _weights(5, hidden, hq, hkv)
    x = np.random.default_rng(6).standard_normal((b, n, hidden))
    out, kc, vc, (q, k, v), attn = ol.qwen3_attention_layer(x, w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base,
                                                            schedule=schedule, return_heads=True)
    bf, _ = oracle.bifocal_bruteforce(q, k, v, big_l, w, base, schedule=schedule)
    assert np.abs(attn - bf).max() <= 1e-12
    assert np.abs(out - bf.reshape(b, n, hq * D) @ w_o.T).max() <= 1e-12
    # and it is not the base model
    plain, _, _ = ol.qwen3_attention_layer(x, w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base, bifocal=False)
    assert np.abs(out - plain).max() > 1e-4


def test_layer_in_two_chunks_equals_one_call():
    # the second chunk sees s = 90, like the single call, so g is the same
    b, hidden, hq, hkv, big_l, w, base = 2, 64, 4, 2, 32, 8, 1e4
    w_qkv, gq, gk, w_o = _weights(7, hidden, hq, hkv)
    x = np.random.default_rng(8).standard_normal((b, 90, hidden))
    full, kf, vf = ol.qwen3_attention_layer(x, w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base)
    _, k1, v1 = ol.qwen3_attention_layer(x[:, :61], w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base)
    out2, k2, v2 = ol.qwen3_attention_layer(x[:, 61:], w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base, k1, v1)
    assert np.abs(out2 - full[:, 61:]).max() <= 1e-12
    assert np.abs(k2 - kf).max() <= 1e-12 and np.abs(v2 - vf).max() <= 1e-12


def test_layer_row_subset_matches_full():
    b, hidden, hq, hkv, big_l, w, base = 1, 64, 4, 2, 16, 5, 1e4
    w_qkv, gq, gk, w_o = _weights(9, hidden, hq, hkv)
    x = np.random.default_rng(10).standard_normal((b, 50, hidden))
    rows = np.array([0, 4, 5, 17, 49])
    for bif in (True, False):
        full, _, _ = ol.qwen3_attention_layer(x, w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base, bifocal=bif)
        part, _, _ = ol.qwen3_attention_layer(x, w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base, bifocal=bif, rows=rows)
        assert np.abs(part - full[:, rows]).max() <= 1e-13
