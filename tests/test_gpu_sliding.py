"""GPU parity of the sliding-window prefill and decode against the fp64 oracle.

Sliding-window layers sit next to the global ones in hybrid models
(seventnews.com, "Generalization to hybrid attention architectures"); a window
W <= L never leaves the pretrained positions, so they are plain attention over
the newest W keys of each row -- the local view of the bifocal merge.  Shapes
span ragged tails, GQA groups, a chunk of queries, W = 1, windows of one tile
and windows wider than the context.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv, normal_bf16

from gpu_helpers import LSE_MEAN_TOL, LSE_TOL_PLAIN, assert_parity, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu


def _prefill(qb, kb, vb, w, plain=False):
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    b, n_q, hq, _ = qb.shape
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, n_q), dtype=torch.float32, device="cuda:0")
    print(f"sliding prefill B={b} n_q={n_q} n_kv={kb.shape[1]} Hq={hq} Hkv={kb.shape[2]} W={w} plain={plain}",
          flush=True)
    if plain:
        jl.jl_plain_prefill(q, k, v, out, lse)
    else:
        jl.jl_sliding_prefill(q, k, v, out, lse, w)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


CASES = [
    # workload id, B, n_q, n_kv, Hq, Hkv, W
    (400, 1, 2048, 2048, 1, 1, 128),
    (401, 1, 300, 300, 4, 2, 40),       # ragged, G = 2
    (402, 1, 77, 500, 4, 1, 32),        # a chunk of 77 queries at the end of 500 keys
    (403, 2, 200, 200, 2, 2, 1),        # W = 1: each row is its own value
    (404, 1, 700, 700, 8, 1, 64),       # a window of exactly one tile
    (405, 1, 513, 513, 4, 4, 65),       # one key past a tile
    (406, 1, 1000, 1000, 16, 4, 256),
    (407, 1, 1500, 1500, 4, 2, 700),    # wide window: many tiles inside every row's window, unmasked
]


@pytest.mark.parametrize("case", CASES, ids=[f"w{c[0]}" for c in CASES])
def test_sliding_prefill_parity(case):
    wid, b, n_q, n_kv, hq, hkv, w = case
    qb, kb, vb = make_qkv(wid, b, n_q, n_kv, hq, hkv, 128)
    out, lse = _prefill(qb, kb, vb, w)
    ro, rl = oracle.sliding_window_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), w)
    assert_parity(out, ro, f"sliding prefill {case}")
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)


def test_sliding_prefill_wide_window_is_plain():
    qb, kb, vb = make_qkv(410, 1, 900, 900, 4, 2, 128)
    out, lse = _prefill(qb, kb, vb, 5000)
    out_p, lse_p = _prefill(qb, kb, vb, 0, plain=True)
    assert_parity(out, out_p, "window wider than the context vs plain", max_tol=2e-3, mean_tol=1e-4)
    assert_parity(lse, lse_p, "lse", max_tol=1e-4, mean_tol=1e-5)


def test_sliding_prefill_full_size_sampled_rows():
    # Qwen3-8B-shaped layer at 128K with a 4096-key window (32 / 8 heads, D 128)
    n, hq, hkv, w = 131072, 32, 8, 4096
    qb, kb, vb = make_qkv(420, 1, n, n, hq, hkv, 128)
    out, lse = _prefill(qb, kb, vb, w)
    rows = sample_rows(n, n, 32768, w, 4, count=24, seed=3)
    ro, rl = oracle.sliding_window_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), w,
                                             rows=rows)
    assert_parity(out[:, rows], ro, "sliding prefill 128K sampled rows")
    assert_parity(lse[:, :, rows], rl, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)


def _decode(q, kc, vc, w, plain=False):
    b, _, hq, _ = q.shape
    n_kv, hkv = kc.shape[1], kc.shape[2]
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, 1), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(jl.jl_bifocal_decode_workspace_size(b, n_kv, hq, hkv), dtype=torch.uint8, device="cuda:0")
    print(f"sliding decode B={b} n_kv={n_kv} Hq={hq} Hkv={hkv} W={w} plain={plain}", flush=True)
    if plain:
        jl.jl_plain_decode(q, kc, vc, out, lse, ws)
    else:
        jl.jl_sliding_decode(q, kc, vc, out, lse, w, ws)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("n_kv,w", [(1, 16), (127, 128), (2200, 128), (2200, 1), (3000, 1024), (32768, 4096),
                                    (131072, 4096)])
def test_sliding_decode_parity(n_kv, w):
    hq, hkv = (32, 8) if n_kv >= 32768 else (8, 2)
    qb = normal_bf16(430, n_kv, (2 if n_kv < 32768 else 1, 1, hq, 128))
    kb = normal_bf16(431, n_kv, (qb.shape[0], n_kv, hkv, 128))
    vb = normal_bf16(432, n_kv, (qb.shape[0], n_kv, hkv, 128))
    out, lse = _decode(to_device(qb), to_device(kb), to_device(vb), w)
    lo = max(0, n_kv - w)  # only the window's keys enter: the oracle sees the full cache
    ro, rl = oracle.sliding_window_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), w)
    assert_parity(out, ro, f"sliding decode n_kv={n_kv} W={w} (keys {lo}..{n_kv - 1})")
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)


def test_sliding_decode_wide_window_is_plain_bitwise_and_matches_prefill_row():
    qb, kb, vb = make_qkv(440, 1, 700, 700, 4, 2, 128)
    q, kc, vc = to_device(qb), to_device(kb), to_device(vb)
    qd = q[:, -1:].contiguous()
    a = _decode(qd, kc, vc, 700)
    p = _decode(qd, kc, vc, 0, plain=True)
    assert np.array_equal(a[0], p[0]) and np.array_equal(a[1], p[1])
    out, _ = _prefill(qb, kb, vb, 100)
    dec, _ = _decode(qd, kc, vc, 100)
    assert_parity(dec, out[:, -1:], "sliding decode vs prefill last row", max_tol=1e-2, mean_tol=1e-3)
