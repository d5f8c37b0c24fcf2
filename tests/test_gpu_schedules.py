"""GPU parity of the long-range schedule variants against the fp64 oracle.

The long-range branch rescales positions by a factor that follows the current
length, and the method is reported robust across rescaling schedules
(seventnews.com, "How bifocal attention sidesteps the fixed-scaling trap").
Besides the integer grouping every other test covers, the kernels run the
seam-shifted grouping (remote distances continue the local ones) and the
fractional scaling (remote positions p / l, l real); the oracle's
``long_range_schedule`` states both.  The integer grouping through the
schedule entry points must be bitwise the result of the plain entry points.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv, normal_bf16

from gpu_helpers import LSE_MEAN_TOL, LSE_TOL, assert_parity, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

VARIANTS = ["seam", "fractional"]
BF16_NAN = np.uint16(0x7FC0)

PREFILL_CASES = [
    # workload id, B, n_q, n_kv, Hq, Hkv, L, W, base
    (200, 1, 1000, 1000, 4, 2, 256, 64, 1e4),    # seam g = 5 (grouped 4), l = 999/255
    (201, 1, 77, 700, 8, 2, 128, 100, 1e6),      # a chunk of 77 queries, W close to L (seam g = 22)
    (202, 2, 300, 300, 2, 2, 64, 1, 1e4),        # W = 1: the shift is 1 once g > 1
    (203, 1, 513, 513, 4, 4, 512, 64, 1e6),      # s = L + 1: the smallest factors above 1
]


def _prefill(case, schedule, two_launch):
    wid, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    qb, kb, vb = make_qkv(wid, b, n_q, n_kv, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, n_q), dtype=torch.float32, device="cuda:0")
    ws = None
    if two_launch:
        ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(b, n_kv, hkv), dtype=torch.uint8, device="cuda:0")
    print(f"prefill schedule={schedule} two_launch={two_launch} case={case}", flush=True)
    jl.jl_bifocal_prefill_sched(q, k, v, out, lse, big_l, w, base, schedule, ws)
    torch.cuda.synchronize()
    return (qb, kb, vb), (q, k, v), out, lse


@pytest.mark.parametrize("two_launch", [True, False], ids=["two_launch", "single_kernel"])
@pytest.mark.parametrize("schedule", VARIANTS)
@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"w{c[0]}" for c in PREFILL_CASES])
def test_prefill_schedule_parity(case, schedule, two_launch):
    _, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    (qb, kb, vb), _, out, lse = _prefill(case, schedule, two_launch)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), big_l, w, base,
                                    schedule=schedule)
    assert jl.jl_schedule_factor(n_kv, big_l, w, schedule) == pytest.approx(ref["g"], rel=1e-15)
    assert_parity(to_f64(out), ref["out"])
    assert_parity(lse.cpu().numpy().astype(np.float64), ref["lse"], "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("two_launch", [True, False], ids=["two_launch", "single_kernel"])
def test_grouped_schedule_is_the_default_bitwise(two_launch):
    case = PREFILL_CASES[0]
    _, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    _, (q, k, v), out, lse = _prefill(case, "grouped", two_launch)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    if two_launch:
        ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(b, n_kv, hkv), dtype=torch.uint8, device="cuda:0")
        jl.jl_bifocal_prefill_ws(q, k, v, out2, lse2, big_l, w, base, ws)
    else:
        jl.jl_bifocal_prefill(q, k, v, out2, lse2, big_l, w, base)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)


@pytest.mark.parametrize("schedule", list(oracle.SCHEDULES))
def test_short_input_is_plain_for_every_schedule(schedule):
    # s <= L: every schedule is the base model, computed by the plain kernel bitwise
    case = (204, 1, 400, 400, 4, 2, 512, 64, 1e4)
    _, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    _, (q, k, v), out, lse = _prefill(case, schedule, True)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    jl.jl_plain_prefill(q, k, v, out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)


def _decode(qb, kb, vb, lens, big_l, w, base, schedule, varlen):
    b, _, hq, _ = qb.shape
    n_max, hkv = kb.shape[1], kb.shape[2]
    q, kc, vc = to_device(qb), to_device(kb), to_device(vb)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, 1), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(jl.jl_bifocal_decode_workspace_size(b, n_max, hq, hkv), dtype=torch.uint8, device="cuda:0")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda:0") if varlen else None
    print(f"decode schedule={schedule} lens={list(lens)} n_max={n_max} Hq={hq} Hkv={hkv} L={big_l} W={w} "
          f"varlen={varlen}", flush=True)
    jl.jl_bifocal_decode_sched(q, kc, vc, out, lse, sl, big_l, w, base, schedule, ws)
    torch.cuda.synchronize()
    return (q, kc, vc, ws, sl), out, lse


def _decode_inputs(seed, lens, hq, hkv):
    n_max, b = max(lens), len(lens)
    qb = normal_bf16(seed, 0, (b, 1, hq, 128))
    kb = normal_bf16(seed, 1, (b, n_max, hkv, 128))
    vb = normal_bf16(seed, 2, (b, n_max, hkv, 128))
    for bi, s in enumerate(lens):
        kb[bi, s:] = BF16_NAN
        vb[bi, s:] = BF16_NAN
    return qb, kb, vb


def _decode_oracle(qb, kb, vb, lens, big_l, w, base, schedule):
    q = bf16_bits_to_f64(qb)
    outs, lses = [], []
    for bi, s in enumerate(lens):
        o, l = oracle.bifocal_decode(q[bi:bi + 1], bf16_bits_to_f64(kb[bi:bi + 1, :s]),
                                     bf16_bits_to_f64(vb[bi:bi + 1, :s]), big_l, w, base, schedule=schedule)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


DECODE_CASES = [
    # seed, lens, Hq, Hkv, L, W, base, varlen
    (400, (3000, 3000), 8, 2, 512, 128, 1e4, False),
    (401, (1, 700, 1537, 3000), 8, 2, 512, 128, 1e4, True),     # factors from 1 up, one per sequence
    (402, (513, 2049, 4000), 16, 1, 512, 500, 1e6, True),       # W close to L, G = 16
    (403, (20000,), 32, 8, 4096, 512, 1e6, False),
]


@pytest.mark.parametrize("schedule", VARIANTS)
@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"s{c[0]}" for c in DECODE_CASES])
def test_decode_schedule_parity(case, schedule):
    seed, lens, hq, hkv, big_l, w, base, varlen = case
    qb, kb, vb = _decode_inputs(seed, list(lens), hq, hkv)
    _, out, lse = _decode(qb, kb, vb, lens, big_l, w, base, schedule, varlen)
    ro, rl = _decode_oracle(qb, kb, vb, lens, big_l, w, base, schedule)
    assert_parity(to_f64(out), ro)
    assert_parity(lse.cpu().numpy().astype(np.float64), rl, "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("varlen", [False, True])
def test_grouped_decode_schedule_is_the_default_bitwise(varlen):
    lens = (3000, 3000) if not varlen else (1, 700, 1537, 3000)
    qb, kb, vb = _decode_inputs(410, list(lens), 8, 2)
    (q, kc, vc, ws, sl), out, lse = _decode(qb, kb, vb, lens, 512, 128, 1e4, "grouped", varlen)
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    if varlen:
        jl.jl_bifocal_decode_varlen(q, kc, vc, out2, lse2, sl, 512, 128, 1e4, ws)
    else:
        jl.jl_bifocal_decode(q, kc, vc, out2, lse2, 512, 128, 1e4, ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(lse, lse2)


@pytest.mark.parametrize("schedule", VARIANTS)
def test_full_size_128k_sampled_rows(schedule):
    # the 128K Qwen3-8B-shaped layer (32 / 8 heads, L = 32768, W = 4096) in the
    # two-launch form the bench times; sampled rows of two KV heads
    wid, s, hq, hkv, big_l, w, base = 2, 131072, 32, 8, 32768, 4096, 1e6
    qb, kb, vb = make_qkv(wid, 1, s, s, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out = torch.empty_like(q)
    lse = torch.empty((1, hq, s), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(1, s, hkv), dtype=torch.uint8, device="cuda:0")
    g = int(round(jl.jl_schedule_factor(s, big_l, w, "seam"))) if schedule == "seam" else 4
    print(f"full size 128K prefill schedule={schedule}", flush=True)
    jl.jl_bifocal_prefill_sched(q, k, v, out, lse, big_l, w, base, schedule, ws)
    torch.cuda.synchronize()
    rows = sample_rows(s, s, big_l, w, g, count=16)
    grp = hq // hkv
    kf, vf = bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    for kvh in (0, hkv - 1):
        heads = slice(kvh * grp, (kvh + 1) * grp)
        ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb[:, :, heads]), kf[:, :, kvh:kvh + 1],
                                        vf[:, :, kvh:kvh + 1], big_l, w, base, rows=rows, schedule=schedule)
        assert_parity(to_f64(out[:, rows, heads]), ref["out"], f"128K {schedule} kv head {kvh}")
        got_lse = lse[:, heads][:, :, rows].cpu().numpy().astype(np.float64)
        assert_parity(got_lse, ref["lse"], "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)
    # decode of the next token against the same 128K cache (its last row as the query)
    del out, lse, ws
    qd = q[:, s - 1:s].contiguous()
    outd = torch.empty_like(qd)
    lsed = torch.empty((1, hq, 1), dtype=torch.float32, device="cuda:0")
    wsd = torch.empty(jl.jl_bifocal_decode_workspace_size(1, s, hq, hkv), dtype=torch.uint8, device="cuda:0")
    print(f"full size 128K decode schedule={schedule}", flush=True)
    jl.jl_bifocal_decode_sched(qd, k, v, outd, lsed, None, big_l, w, base, schedule, wsd)
    torch.cuda.synchronize()
    ro, rl = oracle.bifocal_decode(bf16_bits_to_f64(qb[:, s - 1:s]), kf, vf, big_l, w, base, schedule=schedule)
    assert_parity(to_f64(outd), ro, f"128K decode {schedule}")
    assert_parity(lsed.cpu().numpy().astype(np.float64), rl, "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)
