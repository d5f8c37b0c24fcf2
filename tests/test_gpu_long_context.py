"""GPU parity far beyond the 128K workload: a context of 2^20 + 3 keys (a ragged
last tile), where the group factor reaches 33 and the correction angles c(p) theta_0
exceed 10^6 radians.  A chunk of the newest 3000 query rows runs through the
single-kernel and the two-launch prefill, and the newest row through the decode;
sampled rows (both ends of the chunk and random ones, which include rows whose
local window ends inside a tile) are checked against the fp64 oracle with the bar
of every other parity test (max-abs 1e-2, mean-abs 1e-3; lse 4e-3 with g > 1).
With N(0, 1) queries the weight of a row spreads over many of its million keys and
the outputs are small; queries scaled by 4 concentrate it on few keys, so that the
outputs are of order one.  Scores then have a standard deviation of about 4, and
the bf16 rounding of the corrected q^g and k^g moves each grouped score in
proportion to its size, so that case is held to the bar scaled by the same 4 (as
the peaked-score prefill test is): the oracle itself, with q^g and k^g rounded to
bf16 before the products, moves by max-abs 1.2e-2 and mean-abs 9.8e-4 on these
rows (lse 1.2e-2 / 3.4e-3).
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, normal_bf16

from gpu_helpers import LSE_MEAN_TOL, MAX_ABS_TOL, MEAN_ABS_TOL, assert_parity, lse_tol, to_device, to_f64

pytestmark = pytest.mark.gpu

N_KV = (1 << 20) + 3
N_Q = 3000
HQ, HKV = 4, 1
BIG_L, W, BASE = 32768, 4096, 1e6


@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_long_context_chunk_prefill_and_decode(q_scale):
    print(f"case long context: n_kv={N_KV} n_q={N_Q} Hq={HQ} Hkv={HKV} L={BIG_L} W={W} base={BASE} "
          f"q_scale={q_scale}", flush=True)
    qb = normal_bf16(950, 0, (1, N_Q, HQ, 128), q_scale)
    kb = normal_bf16(950, 1, (1, N_KV, HKV, 128))
    vb = normal_bf16(950, 2, (1, N_KV, HKV, 128))
    rng = np.random.default_rng(950)
    rows = np.unique(np.concatenate([np.arange(4), np.arange(N_Q - 4, N_Q), rng.choice(N_Q, 8, replace=False)]))
    g = jl.jl_group_factor(N_KV, BIG_L)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), BIG_L, W, BASE,
                                    rows=rows, row_block=8)
    assert ref["g"] == g == 33
    bar = q_scale  # the parity bar scaled with the scores
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(1, N_KV, HKV), dtype=torch.uint8, device="cuda:0")
    for form in ("single_kernel", "two_launch"):
        out = torch.empty_like(q)
        lse = torch.empty((1, HQ, N_Q), dtype=torch.float32, device="cuda:0")
        if form == "single_kernel":
            jl.jl_bifocal_prefill(q, k, v, out, lse, BIG_L, W, BASE)
        else:
            jl.jl_bifocal_prefill_ws(q, k, v, out, lse, BIG_L, W, BASE, ws)
        torch.cuda.synchronize()
        print(f"long context prefill, {form}", flush=True)
        got = to_f64(out[:, rows])
        print(f"output magnitude: max {np.abs(ref['out']).max():.3f}, mean {np.abs(ref['out']).mean():.3f}", flush=True)
        assert_parity(got, ref["out"], f"prefill {form}", max_tol=MAX_ABS_TOL * bar, mean_tol=MEAN_ABS_TOL * bar)
        assert_parity(lse[:, :, rows].cpu().numpy().astype(np.float64), ref["lse"], "lse", max_tol=lse_tol(g) * bar,
                      mean_tol=LSE_MEAN_TOL * bar)
    # decode: the newest row (position N_KV - 1) against the whole cache
    qd = q[:, N_Q - 1:].contiguous()
    od = torch.empty_like(qd)
    ld = torch.empty((1, HQ, 1), dtype=torch.float32, device="cuda:0")
    dws = torch.empty(jl.jl_bifocal_decode_workspace_size(1, N_KV, HQ, HKV), dtype=torch.uint8, device="cuda:0")
    jl.jl_bifocal_decode(qd, k, v, od, ld, BIG_L, W, BASE, dws)
    torch.cuda.synchronize()
    assert rows[-1] == N_Q - 1
    assert_parity(to_f64(od), ref["out"][:, -1:], "decode", max_tol=MAX_ABS_TOL * bar, mean_tol=MEAN_ABS_TOL * bar)
    assert_parity(ld.cpu().numpy().astype(np.float64), ref["lse"][:, :, -1:], "decode lse",
                  max_tol=lse_tol(g) * bar, mean_tol=LSE_MEAN_TOL * bar)
