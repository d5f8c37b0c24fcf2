"""GPU parity of the prefill with explicit query positions against the fp64 oracle.

The cache keeps original positions (ResearchPod transcript, cache exchange), so a
call may score query rows at any positions of the context: row i at q_pos[i]
(sorted, with gaps or repeats), with g from the context length.  Each row must be
the whole prefill's row at that position.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv

from gpu_helpers import LSE_MEAN_TOL, LSE_TOL, LSE_TOL_PLAIN, assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run(wid, b, n_kv, hq, hkv, pos, big_l=None, w=None, base=None, schedule="grouped", plain=False, form="fused"):
    n_q = len(pos)
    qb, kb, vb = make_qkv(wid, b, n_q, n_kv, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, n_q), dtype=torch.float32, device="cuda:0")
    qp = torch.tensor(pos, dtype=torch.int32, device="cuda:0")
    print(f"prefill positions wid={wid} B={b} n_q={n_q} n_kv={n_kv} Hq={hq} Hkv={hkv} L={big_l} W={w} "
          f"schedule={schedule} plain={plain} form={form}", flush=True)
    if plain:
        jl.jl_plain_prefill(q, k, v, out, lse, q_pos=qp)
    elif form == "fused" and schedule == "grouped":
        jl.jl_bifocal_prefill(q, k, v, out, lse, big_l, w, base, q_pos=qp)
    elif form == "fused":
        jl.jl_bifocal_prefill_positions(q, k, v, out, lse, qp, big_l, w, base, None, schedule=schedule)
    else:
        ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(b, n_kv, hkv), dtype=torch.uint8, device="cuda:0")
        jl.jl_bifocal_prefill_positions(q, k, v, out, lse, qp, big_l, w, base, ws, schedule=schedule)
    torch.cuda.synchronize()
    return (qb, kb, vb), (q, k, v, qp), to_f64(out), lse.cpu().numpy().astype(np.float64)


def _positions(seed, n_kv, n_q):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(n_kv, n_q, replace=True)).astype(np.int64)


CASES = [
    # wid, B, n_kv, n_q, Hq, Hkv, L, W, base
    (700, 1, 1000, 300, 4, 2, 256, 64, 1e4),     # g = 4; gaps and repeats
    (701, 2, 700, 97, 8, 2, 128, 100, 1e6),      # batch 2, W close to L
    (702, 1, 2048, 64, 4, 4, 512, 128, 1e4),     # one query block spread over the whole context
    (703, 1, 1500, 400, 4, 2, 600, 520, 1e4),    # wide window: unmasked local tiles below each block's rows
]


FORMS = ["fused", "two_launch"]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("case", CASES, ids=[f"w{c[0]}" for c in CASES])
def test_prefill_positions_parity(case, form):
    wid, b, n_kv, n_q, hq, hkv, big_l, w, base = case
    pos = _positions(wid, n_kv, n_q)
    (qb, kb, vb), _, out, lse = _run(wid, b, n_kv, hq, hkv, pos, big_l, w, base, form=form)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), big_l, w, base,
                                    positions=pos)
    assert_parity(out, ref["out"])
    assert_parity(lse, ref["lse"], "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("schedule", ["seam", "fractional"])
def test_prefill_positions_schedules(schedule, form):
    pos = _positions(710, 1200, 250)
    (qb, kb, vb), _, out, lse = _run(710, 1, 1200, 4, 2, pos, 256, 64, 1e4, schedule=schedule, form=form)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), 256, 64, 1e4,
                                    positions=pos, schedule=schedule)
    assert_parity(out, ref["out"])
    assert_parity(lse, ref["lse"], "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


def test_plain_prefill_positions_parity():
    pos = _positions(720, 900, 333)
    (qb, kb, vb), _, out, lse = _run(720, 1, 900, 8, 2, pos, plain=True)
    ro, rl = oracle.plain_causal_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb),
                                           positions=pos)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("form", ["plain"] + FORMS)
def test_newest_positions_match_the_default_call(form):
    # q_pos = n_kv - n_q + i is the call without positions: the same sweep, the same
    # corrected keys and the same rounding, so bit for bit in every form
    plain = form == "plain"
    n_kv, n_q = 1000, 400
    pos = np.arange(n_kv - n_q, n_kv)
    _, (q, k, v, _), out, lse = _run(730, 1, n_kv, 8, 2, pos, 256, 64, 1e4, plain=plain, form=form)
    out2 = torch.empty_like(q)
    lse2 = torch.empty((1, 8, n_q), dtype=torch.float32, device="cuda:0")
    if plain:
        jl.jl_plain_prefill(q, k, v, out2, lse2)
    elif form == "fused":
        jl.jl_bifocal_prefill(q, k, v, out2, lse2, 256, 64, 1e4)
    else:
        ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(1, n_kv, 2), dtype=torch.uint8, device="cuda:0")
        jl.jl_bifocal_prefill_ws(q, k, v, out2, lse2, 256, 64, 1e4, ws)
    torch.cuda.synchronize()
    o2, l2 = to_f64(out2), lse2.cpu().numpy().astype(np.float64)
    n_diff = np.count_nonzero(o2 != out)
    print(f"positions vs default: out differs in {n_diff} of {out.size}, max {np.abs(o2 - out).max():.3e}", flush=True)
    assert n_diff == 0 and np.array_equal(l2, lse)


@pytest.mark.parametrize("form", FORMS)
def test_prefill_positions_128k_sampled(form):
    # 1024 query rows spread over the 128K Qwen3-8B-shaped context (g = 4); sampled
    # rows of two KV heads against the oracle
    n_kv, hq, hkv, big_l, w, base = 131072, 32, 8, 32768, 4096, 1e6
    pos = np.sort(np.concatenate([np.arange(0, n_kv, 128), [4095, 4096, 32767, 32768, n_kv - 1]]))[:1024]
    pos = np.sort(np.unique(np.concatenate([pos[:1019], [4095, 4096, 32767, 32768, n_kv - 1]])))
    (qb, kb, vb), _, out, lse = _run(740, 1, n_kv, hq, hkv, pos, big_l, w, base, form=form)
    rows = np.unique(np.concatenate([[0, 1, len(pos) // 2, len(pos) - 1], np.searchsorted(pos, [4095, 4096, 32768])]))
    kf, vf = bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    grp = hq // hkv
    for kvh in (0, hkv - 1):
        heads = slice(kvh * grp, (kvh + 1) * grp)
        ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb[:, :, heads]), kf[:, :, kvh:kvh + 1], vf[:, :, kvh:kvh + 1],
                                        big_l, w, base, rows=rows, positions=pos)
        assert_parity(out[:, rows][:, :, heads], ref["out"], f"128K positions kv head {kvh}")
        assert_parity(lse[:, heads][:, :, rows], ref["lse"], "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)
