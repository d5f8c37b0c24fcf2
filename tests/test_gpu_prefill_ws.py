"""GPU parity of the two-launch bifocal prefill (corrected keys precomputed into
a caller workspace, then staged like plain keys) against the fp64 oracle.

Same cases and bar as the fused path (max-abs <= 1e-2, mean-abs <= 1e-3), plus
workspace reuse across calls of different sizes and the g = 1 short-circuit (no
workspace needed).  The full workload sizes are checked for both forms in
test_gpu_full_sizes."""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv

from gpu_helpers import LSE_MEAN_TOL, assert_parity, lse_tol, to_device, to_f64
from test_gpu_prefill import CASES

pytestmark = pytest.mark.gpu


def _workspace(b, n_kv, hkv):
    nbytes = jl.jl_bifocal_prefill_workspace_size(b, n_kv, hkv)
    assert nbytes == b * n_kv * hkv * 128 * 2
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")


def _run_ws(workload, b, n_q, n_kv, hq, hkv, big_l, w, base, ws=None):
    qb, kb, vb = make_qkv(workload, b, n_q, n_kv, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, n_q), dtype=torch.float32, device="cuda:0")
    if ws is None:
        ws = _workspace(b, n_kv, hkv)
    print(f"ws case workload={workload} B={b} n_q={n_q} n_kv={n_kv} Hq={hq} Hkv={hkv} L={big_l} W={w}", flush=True)
    jl.jl_bifocal_prefill_ws(q, k, v, out, lse, big_l, w, base, ws)
    torch.cuda.synchronize()
    return (qb, kb, vb), to_f64(out), lse.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", CASES, ids=[f"w{c[0]}" for c in CASES])
def test_ws_prefill_parity(case):
    wid, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    (qb, kb, vb), out, lse = _run_ws(wid, b, n_q, n_kv, hq, hkv, big_l, w, base)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), big_l, w, base)
    assert_parity(out, ref["out"])
    assert_parity(lse, ref["lse"], "lse", max_tol=lse_tol(ref["g"]), mean_tol=LSE_MEAN_TOL)


def test_ws_workspace_reused_with_smaller_problem():
    # one workspace, a large call then a smaller one: the second reads only what it wrote
    ws = _workspace(1, 2048, 2)
    for case in [(130, 1, 2048, 2048, 4, 2, 512, 128, 1e4), (131, 1, 300, 700, 4, 2, 128, 40, 1e6)]:
        wid, b, n_q, n_kv, hq, hkv, big_l, w, base = case
        (qb, kb, vb), out, lse = _run_ws(wid, b, n_q, n_kv, hq, hkv, big_l, w, base, ws=ws)
        ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), big_l, w,
                                        base)
        assert_parity(out, ref["out"])


def test_ws_short_input_needs_no_workspace_and_is_plain():
    qb, kb, vb = make_qkv(132, 1, 500, 500, 4, 2, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out, out_p = torch.empty_like(q), torch.empty_like(q)
    jl.jl_bifocal_prefill_ws(q, k, v, out, None, 512, 64, 1e4, None)  # g = 1
    jl.jl_plain_prefill(q, k, v, out_p, None)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_p.view(torch.int16))
