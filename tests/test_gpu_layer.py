"""GPU parity of the Qwen3-shaped attention layer against the fp64 oracle.

Values enter the cache as the projection gives them, rounded once to bf16
(|error| <= 2^-8 |v|, bf16's unit roundoff, plus fp32 accumulation noise); keys
are checked against the bound their two bf16 roundings give.

The layer (projection, per-head RMSNorm, RoPE and cache append, bifocal or
plain attention, output projection) runs as one C call; the oracle states the
same layer in fp64 (oracle.layer).  The output projection's weights have
N(0, 1/fan_in) entries, so it carries the attention's absolute error to the
output at about the same size: the attention's bar (max-abs 1e-2, mean-abs
1e-3) applies to the layer output, plus the two bf16 roundings the attention
bar does not see (the attention output and the layer output, each up to 2^-8
of the value, the former carried to the output at about the output's size):
|error| <= 1e-2 + 2^-7 |out| per element, mean-abs <= 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_layer

from gpu_helpers import assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu



def _device_layer(wid, b, n_total, hidden, hq, hkv):
    x, w_qkv, w_o, gq, gk = make_layer(wid, b, n_total, hidden, hq, hkv)
    host = tuple(bf16_bits_to_f64(a) for a in (x, w_qkv, w_o, gq, gk))
    dev = tuple(to_device(a) for a in (x, w_qkv, w_o, gq, gk))
    return host, dev


def _run_chunks(dev, b, chunks, hq, hkv, bifocal, big_l, w, base, schedule="grouped"):
    """Run the GPU layer over consecutive chunks of the tokens, appending to one
    cache; returns the outputs of every chunk, concatenated, and the caches."""
    x, w_qkv, w_o, gq, gk = dev
    n_total, hidden = x.shape[1], x.shape[2]
    kc = torch.full((b, n_total, hkv, 128), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    vc = torch.full_like(kc, float("nan"))
    outs = []
    start = 0
    for n in chunks:
        n_kv = start + n
        xs = x[:, start:n_kv].contiguous()
        out = torch.empty((b, n, hidden), dtype=torch.bfloat16, device="cuda:0")
        ws = torch.empty(jl.jl_qwen3_layer_workspace_size(b, n, n_kv, hq, hkv), dtype=torch.uint8, device="cuda:0")
        # the call sees only the first n_kv rows of the cache
        k_view, v_view = kc[:, :n_kv].contiguous(), vc[:, :n_kv].contiguous()
        print(f"layer chunk [{start}, {n_kv}) B={b} hidden={hidden} Hq={hq} Hkv={hkv} bifocal={bifocal} "
              f"L={big_l} W={w} schedule={schedule}", flush=True)
        jl.jl_qwen3_attention_layer(xs, w_qkv, gq, gk, w_o, out, k_view, v_view, ws, bifocal=bifocal,
                                    pretrained_window=big_l, local_window=w, rope_base=base, schedule=schedule)
        torch.cuda.synchronize()
        kc[:, :n_kv].copy_(k_view)
        vc[:, :n_kv].copy_(v_view)
        outs.append(out)
        start = n_kv
    return torch.cat(outs, dim=1), kc, vc


def _assert_keys(got, ref):
    # A key element is a rotation of a pair (u_d, u_d+64) of normalised projected
    # values, each rounded to bf16 once before (relative 2^-8) and the result once
    # after: |error| <= 2^-8 (sqrt(2) + 1 + 1) r with r the pair's norm (the third
    # term for the norm's own scale), i.e. at most 2^-6.2 r; checked against 2^-6 r
    # plus fp32 noise.
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    r = np.sqrt(ref[..., :64] ** 2 + ref[..., 64:] ** 2)
    bound = 2.0 ** -6 * np.concatenate([r, r], axis=-1) + 1e-4
    print(f"k cache: worst error / bound {np.max(err / bound):.3f}, mean-abs {err.mean():.2e}", flush=True)
    assert np.all(err <= bound)


def _assert_values(got, ref):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5
    print(f"v cache: worst error / bound {np.max(err / bound):.3f}", flush=True)
    assert np.all(np.isfinite(got)) and np.all(err <= bound)


def _assert_out(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bound = 1e-2 + 2.0 ** -7 * np.abs(ref)
    print(f"{what}: max-abs {err.max():.3e}, worst error / bound {np.max(err / bound):.3f}, "
          f"mean-abs {err.mean():.3e} (tol 1e-3)", flush=True)
    assert np.all(err <= bound) and err.mean() <= 1e-3

CASES = [
    # workload id, B, chunks, hidden, Hq, Hkv, bifocal, L, W, base, schedule
    (500, 1, (700,), 256, 4, 2, True, 256, 64, 1e4, "grouped"),          # g = 3
    (501, 2, (300, 213, 1), 384, 8, 2, True, 128, 40, 1e6, "grouped"),    # prefill, chunk, then a decode step
    (502, 1, (640,), 256, 4, 4, False, 1, 1, 1e4, "grouped"),             # the plain layer
    (503, 1, (500, 1), 256, 4, 2, True, 128, 32, 1e4, "seam"),
    (504, 1, (500, 1), 256, 4, 2, True, 128, 32, 1e4, "fractional"),
    (507, 5, (200, 1), 256, 4, 2, True, 128, 32, 1e4, "grouped"),      # a decode step of 5 tokens
    (508, 9, (300, 1), 256, 4, 2, True, 128, 32, 1e4, "seam"),        # 9 tokens: past the few-token kernel
]


@pytest.mark.parametrize("case", CASES, ids=[f"w{c[0]}" for c in CASES])
def test_layer_parity(case):
    wid, b, chunks, hidden, hq, hkv, bif, big_l, w, base, schedule = case
    n_total = sum(chunks)
    (x, w_qkv, w_o, gq, gk), dev = _device_layer(wid, b, n_total, hidden, hq, hkv)
    out, kc, vc = _run_chunks(dev, b, chunks, hq, hkv, bif, big_l, w, base, schedule)
    # the oracle runs the same chunks (each chunk's g comes from its own n_kv)
    ref_outs, pk, pv = [], None, None
    start = 0
    for n in chunks:
        o, pk, pv = oracle.qwen3_attention_layer(x[:, start:start + n], w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base,
                                                 pk, pv, bifocal=bif, schedule=schedule)
        ref_outs.append(o)
        start += n
    ref = np.concatenate(ref_outs, axis=1)
    _assert_out(to_f64(out), ref, "layer out")
    _assert_keys(to_f64(kc), pk)
    _assert_values(to_f64(vc), pv)


def test_layer_qwen3_8b_shape_sampled_rows():
    # Qwen3-8B's layer shape (hidden 4096, 32 / 8 heads) at 4096 tokens with
    # L = 1024, W = 256 (g = 4); sampled rows of the output, the whole caches
    wid, b, n, hidden, hq, hkv, big_l, w, base = 505, 1, 4096, 4096, 32, 8, 1024, 256, 1e6
    (x, w_qkv, w_o, gq, gk), dev = _device_layer(wid, b, n, hidden, hq, hkv)
    out, kc, vc = _run_chunks(dev, b, (n,), hq, hkv, True, big_l, w, base)
    rows = np.array([0, 1, 255, 256, 257, 1023, 1024, 2047, 2048, 3000, 4095])
    ref, rk, rv = oracle.qwen3_attention_layer(x, w_qkv, gq, gk, w_o, hq, hkv, big_l, w, base, rows=rows)
    _assert_out(to_f64(out[:, rows]), ref, "layer out (sampled rows)")
    _assert_keys(to_f64(kc), rk)
    _assert_values(to_f64(vc), rv)


def test_plain_and_bifocal_layers_agree_within_the_window():
    # s <= L: the bifocal layer runs the plain kernels, bitwise
    (x, *_), dev = _device_layer(506, 1, 400, 256, 4, 2)
    o1, k1, v1 = _run_chunks(dev, 1, (400,), 4, 2, True, 512, 64, 1e4)
    o2, k2, v2 = _run_chunks(dev, 1, (400,), 4, 2, False, 1, 1, 1e4)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
