"""GPU parity of the variable-length prefill against the fp64 oracle.

Each sequence of a batch brings its own chunk of new query rows (packed) against
its own cache prefix, and gets the factor of its own length: the cache keeps
original positions and the factor follows the current length (ResearchPod
transcript, cache exchange; seventnews.com, "How bifocal attention sidesteps the
fixed-scaling trap").  Cache rows past a sequence's length are NaN in every test:
a read beyond the prefix would poison that sequence's output.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, normal_bf16

from gpu_helpers import LSE_MEAN_TOL, LSE_TOL, LSE_TOL_PLAIN, assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)


def _inputs(seed, spec, hq, hkv, n_max=None):
    """spec: [(new rows n_b, keys s_b)] -> packed q bits, padded cache bits, cu_seqlens"""
    n_max = n_max or max(s for _, s in spec)
    cu = np.concatenate([[0], np.cumsum([n for n, _ in spec])]).astype(np.int32)
    qb = normal_bf16(seed, 0, (int(cu[-1]), hq, 128))
    kb = normal_bf16(seed, 1, (len(spec), n_max, hkv, 128))
    vb = normal_bf16(seed, 2, (len(spec), n_max, hkv, 128))
    for bi, (_, s) in enumerate(spec):
        kb[bi, s:] = BF16_NAN
        vb[bi, s:] = BF16_NAN
    return qb, kb, vb, cu


def _run(qb, kb, vb, cu, spec, big_l=None, w=None, base=None, schedule="grouped", plain=False, form="fused"):
    total_q, hq, _ = qb.shape
    b, n_max, hkv = kb.shape[0], kb.shape[1], kb.shape[2]
    q, kc, vc = to_device(qb), to_device(kb), to_device(vb)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((hq, total_q), float("nan"), dtype=torch.float32, device="cuda:0")
    cu_d = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
    sl = torch.tensor([s for _, s in spec], dtype=torch.int32, device="cuda:0")
    max_q = max(n for n, _ in spec)
    print(f"prefill varlen spec={spec} Hq={hq} Hkv={hkv} L={big_l} W={w} schedule={schedule} plain={plain} "
          f"form={form}", flush=True)
    if plain:
        jl.jl_plain_prefill_varlen(q, kc, vc, out, lse, cu_d, sl, max_q)
    else:
        # the single kernel takes no workspace; the two-launch form writes the corrected keys there first
        ws = None if form == "fused" else torch.empty(jl.jl_bifocal_prefill_workspace_size(b, n_max, hkv),
                                                       dtype=torch.uint8, device="cuda:0")
        jl.jl_bifocal_prefill_varlen(q, kc, vc, out, lse, cu_d, sl, max_q, big_l, w, base, ws, schedule=schedule)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64), (q, kc, vc)


def _oracle(qb, kb, vb, cu, spec, big_l, w, base, schedule="grouped", plain=False):
    return oracle.bifocal_prefill_varlen(bf16_bits_to_f64(qb), cu, bf16_bits_to_f64(kb), bf16_bits_to_f64(vb),
                                         [s for _, s in spec], big_l, w, base, schedule=schedule, bifocal=not plain)


CASES = [
    # seed, [(new rows, keys)], Hq, Hkv, L, W, base
    (600, [(300, 300), (77, 500), (1, 333), (513, 1025)], 8, 2, 256, 64, 1e4),   # g = 2, 2, 2, 5
    (601, [(64, 64), (0, 100), (129, 700), (200, 200)], 4, 4, 128, 128, 1e6),    # an empty chunk; W = L
    (602, [(700, 700), (33, 2000)], 16, 2, 512, 100, 1e4),                        # G = 8
    (603, [(50, 50), (400, 400)], 4, 2, 512, 64, 1e4),                            # every s_b <= L: g = 1
    (604, [(900, 900), (257, 1500)], 4, 2, 600, 520, 1e4),                       # wide window, g = 2, 3
]


FORMS = ["fused", "two_launch"]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_prefill_varlen_parity(case, form):
    seed, spec, hq, hkv, big_l, w, base = case
    qb, kb, vb, cu = _inputs(seed, spec, hq, hkv)
    out, lse, _ = _run(qb, kb, vb, cu, spec, big_l, w, base, form=form)
    ro, rl = _oracle(qb, kb, vb, cu, spec, big_l, w, base)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("schedule", ["seam", "fractional"])
def test_prefill_varlen_schedules(schedule, form):
    spec = [(300, 300), (77, 900), (1, 333), (250, 1300)]
    qb, kb, vb, cu = _inputs(610, spec, 8, 2)
    out, lse, _ = _run(qb, kb, vb, cu, spec, 256, 64, 1e4, schedule=schedule, form=form)
    ro, rl = _oracle(qb, kb, vb, cu, spec, 256, 64, 1e4, schedule=schedule)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


def test_plain_prefill_varlen_parity():
    spec = [(300, 300), (77, 500), (0, 10), (513, 1025)]
    qb, kb, vb, cu = _inputs(620, spec, 8, 2)
    out, lse, _ = _run(qb, kb, vb, cu, spec, plain=True)
    ro, rl = _oracle(qb, kb, vb, cu, spec, None, None, None, plain=True)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("form", ["plain"] + FORMS)
def test_equal_lengths_match_the_uniform_call(form):
    # two sequences of 333 new rows over 1000 keys against the padded-batch call of
    # the same form: the same corrected keys, the same sweep and the same rounding
    # (every rotation is written with explicit fused multiply-adds), so bit for bit
    spec = [(333, 1000), (333, 1000)]
    plain = form == "plain"
    qb, kb, vb, cu = _inputs(630, spec, 8, 2)
    out, lse, (q, kc, vc) = _run(qb, kb, vb, cu, spec, 256, 64, 1e4, plain=plain, form=form)
    q_u = q.view(2, 333, 8, 128)
    out_u = torch.empty_like(q_u)
    lse_u = torch.empty((2, 8, 333), dtype=torch.float32, device="cuda:0")
    if plain:
        jl.jl_plain_prefill(q_u, kc, vc, out_u, lse_u)
    elif form == "fused":
        jl.jl_bifocal_prefill(q_u, kc, vc, out_u, lse_u, 256, 64, 1e4)
    else:
        ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(2, 1000, 2), dtype=torch.uint8, device="cuda:0")
        jl.jl_bifocal_prefill_ws(q_u, kc, vc, out_u, lse_u, 256, 64, 1e4, ws)
    torch.cuda.synchronize()
    ou = to_f64(out_u).reshape(666, 8, 128)
    lu = lse_u.cpu().numpy().transpose(1, 0, 2).reshape(8, 666).astype(np.float64)
    n_diff = np.count_nonzero(ou != out)
    print(f"varlen vs uniform: out differs in {n_diff} of {out.size}, max {np.abs(ou - out).max():.3e}; "
          f"lse differs in {np.count_nonzero(lu != lse)}, max {np.abs(lu - lse).max():.3e}", flush=True)
    assert n_diff == 0 and np.array_equal(lu, lse)


@pytest.mark.parametrize("form", FORMS)
def test_prefill_varlen_full_length_sampled(form):
    # the Qwen3-8B decode-head shape: sequences of 16K and 40K keys with chunks of new rows;
    # sampled rows of every sequence against the oracle
    spec = [(4096, 16384), (1000, 40000), (2048, 2048)]
    hq, hkv, big_l, w, base = 32, 8, 8192, 1024, 1e6
    qb, kb, vb, cu = _inputs(640, spec, hq, hkv)
    out, lse, _ = _run(qb, kb, vb, cu, spec, big_l, w, base, form=form)
    kf, vf = bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    for bi, (n, s) in enumerate(spec):
        rows = np.unique(np.clip(np.array([0, 1, n // 2, n - w - 1, n - w, n - 2, n - 1]), 0, n - 1))
        for kvh in (0, hkv - 1):
            heads = slice(kvh * (hq // hkv), (kvh + 1) * (hq // hkv))
            qsel = bf16_bits_to_f64(qb[cu[bi]:cu[bi + 1], heads])[None]
            ref = oracle.bifocal_three_pass(qsel, kf[bi:bi + 1, :s, kvh:kvh + 1], vf[bi:bi + 1, :s, kvh:kvh + 1],
                                            big_l, w, base, rows=rows)
            assert_parity(out[cu[bi] + rows][:, heads][None], ref["out"], f"seq {bi} kv head {kvh}")
            assert_parity(lse[heads][:, cu[bi] + rows][None], ref["lse"], "lse", max_tol=LSE_TOL,
                          mean_tol=LSE_MEAN_TOL)
