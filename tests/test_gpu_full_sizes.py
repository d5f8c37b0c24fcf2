"""GPU parity at the full workload sizes, on sampled rows.

Rows are independent, so the oracle computes a sample of rows exactly (first
rows, rows around p = W, around L and next to multiples of g, the middle, the
last rows, random rows) for a subset of heads, while the GPU runs the whole
problem in the same launch configuration the bench times.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv

from gpu_helpers import LSE_MEAN_TOL, LSE_TOL, assert_parity, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

# workload id, seq, Hq, Hkv, L, W, base
FULL = {
    "qwen3_1p7b_64k": (1, 65536, 16, 8, 32768, 4096, 1e6),
    "qwen3_8b_128k": (2, 131072, 32, 8, 32768, 4096, 1e6),
    "sweep_48k": (4, 49152, 32, 8, 32768, 4096, 1e6),
    "sweep_96k": (4, 98304, 32, 8, 32768, 4096, 1e6),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_rows(name):
    wid, s, hq, hkv, big_l, w, base = FULL[name]
    g = oracle.group_factor(s, big_l)
    print(f"full size {name}: s={s} Hq={hq} Hkv={hkv} g={g}", flush=True)
    qb, kb, vb = make_qkv(wid, 1, s, s, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out = torch.empty_like(q)
    lse = torch.empty((1, hq, s), dtype=torch.float32, device="cuda:0")
    jl.jl_bifocal_prefill(q, k, v, out, lse, big_l, w, base)
    torch.cuda.synchronize()
    rows = sample_rows(s, s, big_l, w, g, count=20)
    grp = hq // hkv
    kf, vf = bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    for kvh in (0, hkv - 1):
        heads = slice(kvh * grp, (kvh + 1) * grp)
        ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb[:, :, heads]), kf[:, :, kvh:kvh + 1],
                                        vf[:, :, kvh:kvh + 1], big_l, w, base, rows=rows)
        got = to_f64(out[:, rows, heads])
        assert_parity(got, ref["out"], f"{name} kv head {kvh}")
        got_lse = lse[:, heads][:, :, rows].cpu().numpy().astype(np.float64)
        assert_parity(got_lse, ref["lse"], "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("s", [4096, 16384, 32768])
def test_sweep_within_window_is_plain_bitwise(s):
    # length sweep up to the pretrained window: g = 1, the base model exactly
    qb, kb, vb = make_qkv(4, 1, s, s, 32, 8, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out, out_p = torch.empty_like(q), torch.empty_like(q)
    jl.jl_bifocal_prefill(q, k, v, out, None, 32768, 4096, 1e6)
    jl.jl_plain_prefill(q, k, v, out_p, None)
    torch.cuda.synchronize()
    assert torch.equal(out, out_p)
    rows = sample_rows(s, s, 32768, 4096, 1, count=12)
    ref, _ = oracle.plain_causal_attention(bf16_bits_to_f64(qb[:, :, :8]), bf16_bits_to_f64(kb[:, :, :2]),
                                           bf16_bits_to_f64(vb[:, :, :2]), rows=rows)
    assert_parity(to_f64(out[:, rows, :8]), ref, f"sweep {s}")
