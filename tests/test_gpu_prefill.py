"""GPU parity of the fused bifocal prefill against the fp64 oracle.

Every case feeds the HIP path and the oracle the same seeded bf16 inputs and
checks max-abs <= 1e-2 and mean-abs <= 1e-3 on the output (lse within 1e-3).
Shapes span several query blocks and key tiles with ragged tails, GQA groups
of 1/2/4/8, batch > 1, chunks of queries (n_q < n_kv), the degenerate windows
(W = 1, L = 1, W = L) and s on both sides of L.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv

from gpu_helpers import LSE_MEAN_TOL, LSE_TOL_PLAIN, assert_parity, lse_tol, to_device, to_f64

pytestmark = pytest.mark.gpu


def _run(workload, b, n_q, n_kv, hq, hkv, big_l, w, base, q_scale=1.0, plain=False):
    qb, kb, vb = make_qkv(workload, b, n_q, n_kv, hq, hkv, 128, q_scale=q_scale)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, n_q), dtype=torch.float32, device="cuda:0")
    print(f"case workload={workload} B={b} n_q={n_q} n_kv={n_kv} Hq={hq} Hkv={hkv} L={big_l} W={w} "
          f"base={base} q_scale={q_scale} plain={plain}", flush=True)
    if plain:
        jl.jl_plain_prefill(q, k, v, out, lse)
    else:
        jl.jl_bifocal_prefill(q, k, v, out, lse, big_l, w, base)
    torch.cuda.synchronize()
    return (qb, kb, vb), (q, k, v), to_f64(out), lse.cpu().numpy().astype(np.float64)


CASES = [
    # workload id, B, n_q, n_kv, Hq, Hkv, L, W, base
    (100, 1, 2048, 2048, 1, 1, 512, 128, 1e4),    # causal prefill, 1 head, seq 2048 (g = 4)
    (101, 1, 300, 300, 4, 2, 64, 40, 1e4),        # ragged, G = 2, g = 5
    (102, 1, 77, 500, 4, 1, 128, 32, 1e6),        # chunk of 77 queries at the end of 500 keys, G = 4
    (103, 1, 700, 700, 8, 1, 256, 100, 1e4),      # G = 8, g = 3
    (104, 2, 200, 200, 2, 2, 50, 50, 1e4),        # batch 2, W == L, g = 4
    (105, 1, 130, 130, 1, 1, 1, 1, 1e4),          # L = W = 1: g = 130, every remote key aliases to 0
    (106, 1, 513, 513, 4, 4, 512, 64, 1e6),       # s = L + 1 -> g = 2
    (107, 1, 1, 333, 4, 2, 100, 7, 1e4),          # one query row (decode-shaped prefill)
    (108, 1, 1000, 1000, 16, 4, 128, 128, 1e6),   # G = 4 with 4 KV heads, g = 8
    (109, 1, 1500, 1500, 4, 2, 600, 520, 1e4),    # wide window: up to 7 unmasked local tiles per block, g = 3
]


@pytest.mark.parametrize("case", CASES, ids=[f"w{c[0]}" for c in CASES])
def test_bifocal_prefill_parity(case):
    wid, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    (qb, kb, vb), _, out, lse = _run(wid, b, n_q, n_kv, hq, hkv, big_l, w, base)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), big_l, w, base)
    assert ref["g"] == jl.jl_group_factor(n_kv, big_l)
    assert_parity(out, ref["out"])
    assert_parity(lse, ref["lse"], "lse", max_tol=lse_tol(ref["g"]), mean_tol=LSE_MEAN_TOL)


def test_bifocal_prefill_peaked_scores():
    # Q scaled by 4 (score std ~4): a concentrated softmax, where an off-by-one
    # in the local/remote boundary or in g moves the output by far more (max-abs
    # 2.5 for W +- 1, mean-abs 0.4 for g +- 1 in the oracle).  The bf16 rounding
    # of the corrected q^g and k^g moves each grouped score in proportion to its
    # size, so this sensitivity probe is held to the bar scaled by the same 4.
    (qb, kb, vb), _, out, lse = _run(110, 1, 2048, 2048, 1, 1, 512, 128, 1e4, q_scale=4.0)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), 512, 128, 1e4)
    assert_parity(out, ref["out"], max_tol=4e-2, mean_tol=4e-3)
    assert_parity(lse, ref["lse"], "lse", max_tol=4e-2, mean_tol=4e-3)


@pytest.mark.parametrize("case", [(120, 1, 500, 500, 4, 2, 512, 64, 1e4), (121, 2, 96, 640, 8, 2, 640, 640, 1e6)])
def test_short_input_is_plain_attention_bitwise(case):
    # s <= L -> g = 1: the library runs the plain kernel, so results are bitwise
    # equal to jl_plain_prefill, and both match plain attention in the oracle.
    wid, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    assert jl.jl_group_factor(n_kv, big_l) == 1
    (qb, kb, vb), (q, k, v), out, lse = _run(wid, b, n_q, n_kv, hq, hkv, big_l, w, base)
    _, _, out_p, lse_p = _run(wid, b, n_q, n_kv, hq, hkv, big_l, w, base, plain=True)
    assert np.array_equal(out, out_p) and np.array_equal(lse, lse_p)
    ref, ref_lse = oracle.plain_causal_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb))
    assert_parity(out, ref)
    assert_parity(lse, ref_lse, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)


def test_plain_prefill_parity_gqa_ragged():
    (qb, kb, vb), _, out, lse = _run(122, 1, 333, 1000, 8, 2, 1, 1, 1e4, plain=True)
    ref, ref_lse = oracle.plain_causal_attention(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb))
    assert_parity(out, ref)
    assert_parity(lse, ref_lse, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("case", [(130, 1, 2048, 2048, 1, 1, 512, 128, 1e4), (131, 1, 300, 300, 4, 2, 64, 40, 1e4),
                                  (132, 1, 200, 200, 2, 1, 256, 32, 1e4)])
def test_three_passes_match_oracle_passes(case):
    # The per-pass results (A: near keys at base positions, B: all keys folded,
    # C: near keys folded), each against the oracle's pass, plus their merge.
    wid, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    qb, kb, vb = make_qkv(wid, b, n_q, n_kv, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    out_abc = torch.empty((3, b, n_q, hq, 128), dtype=torch.float32, device="cuda:0")
    lse_abc = torch.empty((3, b, hq, n_q), dtype=torch.float32, device="cuda:0")
    jl.jl_bifocal_prefill_passes(q, k, v, out_abc, lse_abc, big_l, w, base)
    torch.cuda.synchronize()
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), big_l, w, base)
    o = out_abc.cpu().numpy().astype(np.float64)
    ls = lse_abc.cpu().numpy().astype(np.float64)
    for i, name in enumerate("ABC"):
        assert_parity(o[i], ref["passes"][name][0], f"pass {name}")
        # pass A scores the vectors as given; B and C score the rounded corrected ones
        tol = LSE_TOL_PLAIN if name == "A" else lse_tol(ref["g"])
        assert_parity(ls[i], ref["passes"][name][1], f"lse {name}", max_tol=tol, mean_tol=LSE_MEAN_TOL)
    merged, merged_lse = oracle.merge_passes(o[0], ls[0], o[1], ls[1], o[2], ls[2])
    assert_parity(merged, ref["out"], "merge of GPU passes")


@pytest.mark.parametrize("case", [(130, 1, 2048, 2048, 1, 1, 512, 128, 1e4), (131, 1, 300, 300, 4, 2, 64, 40, 1e4),
                                  (133, 2, 333, 333, 8, 2, 100, 37, 1e6), (134, 1, 64, 64, 2, 1, 64, 16, 1e4),
                                  (135, 1, 90, 400, 4, 1, 128, 128, 1e4)])
def test_three_pass_merge_in_kernel(case):
    # The literal form of the merge: three passes, each with its own maximum and
    # normaliser, combined by their lse weights in the kernel's epilogue.  Against
    # the oracle's merged result, and against the oracle's merge of the same
    # kernel's per-pass outputs, which it must equal up to the output's bf16
    # rounding (half an ulp: 2^-8 relative) and fp32 rounding in the lse.
    wid, b, n_q, n_kv, hq, hkv, big_l, w, base = case
    qb, kb, vb = make_qkv(wid, b, n_q, n_kv, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    print(f"case three-pass merge workload={wid} B={b} n_q={n_q} n_kv={n_kv} Hq={hq} Hkv={hkv} L={big_l} W={w}",
          flush=True)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, n_q), dtype=torch.float32, device="cuda:0")
    jl.jl_bifocal_prefill_three_pass(q, k, v, out, lse, big_l, w, base)
    out_abc = torch.empty((3, b, n_q, hq, 128), dtype=torch.float32, device="cuda:0")
    lse_abc = torch.empty((3, b, hq, n_q), dtype=torch.float32, device="cuda:0")
    jl.jl_bifocal_prefill_passes(q, k, v, out_abc, lse_abc, big_l, w, base)
    torch.cuda.synchronize()
    got, got_lse = to_f64(out), lse.cpu().numpy().astype(np.float64)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), big_l, w, base)
    assert_parity(got, ref["out"], "three-pass merge")
    assert_parity(got_lse, ref["lse"], "lse", max_tol=lse_tol(ref["g"]), mean_tol=LSE_MEAN_TOL)
    o = out_abc.cpu().numpy().astype(np.float64)
    ls = lse_abc.cpu().numpy().astype(np.float64)
    merged, merged_lse = oracle.merge_passes(o[0], ls[0], o[1], ls[1], o[2], ls[2])
    assert np.all(np.abs(got - merged) <= np.abs(merged) * 2.0 ** -8 * 1.01 + 1e-6), \
        np.abs(got - merged).max()
    assert np.abs(got_lse - merged_lse).max() <= 1e-4


def test_deterministic_and_causal():
    wid, b, n_q, n_kv, hq, hkv, big_l, w, base = 140, 1, 1100, 1100, 4, 1, 300, 64, 1e4
    qb, kb, vb = make_qkv(wid, b, n_q, n_kv, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    outs = []
    for _ in range(3):
        out = torch.empty_like(q)
        jl.jl_bifocal_prefill(q, k, v, out, None, big_l, w, base)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    # perturb keys/values after position 700: rows 0..700 must not move (bitwise)
    k2, v2 = k.clone(), v.clone()
    k2[:, 701:] = -k2[:, 701:]
    v2[:, 701:] = 3 * v2[:, 701:]
    out2 = torch.empty_like(q)
    jl.jl_bifocal_prefill(q, k2, v2, out2, None, big_l, w, base)
    torch.cuda.synchronize()
    assert torch.equal(out2[:, :701], outs[0][:, :701])
    assert not torch.equal(out2[:, 701:], outs[0][:, 701:])


def test_rows_without_remote_keys_match_plain():
    wid, b, n_q, n_kv, hq, hkv, big_l, w, base = 141, 1, 900, 900, 2, 1, 200, 150, 1e4
    _, _, out, _ = _run(wid, b, n_q, n_kv, hq, hkv, big_l, w, base)
    _, _, out_p, _ = _run(wid, b, n_q, n_kv, hq, hkv, big_l, w, base, plain=True)
    # the same keys and scores; the two kernels normalise with different row sums (the
    # single-kernel bifocal form adds the bf16-rounded probabilities, the plain kernel the
    # fp32 ones), which can move an output by one bf16 rounding step
    a, b_ = out[:, :w], out_p[:, :w]
    d = np.abs(a - b_)
    print(f"rows p < W vs plain: max-abs {d.max():.3e}, mean-abs {d.mean():.3e}", flush=True)
    assert np.all(d <= 2.0 ** -7 * np.abs(b_) + 2e-3) and d.mean() <= 1e-4


def test_chunked_prefill_as_the_cache_grows():
    # A prompt prefilled in chunks against the cache so far: each chunk's queries sit at the
    # newest positions and g is taken from the length reached (seventnews.com: the factor follows
    # the current length), so g steps from 1 to 3 across the chunks (L = 512).  Both prefill
    # forms, each chunk against the oracle at its own length.
    big_l, w, base, n, hq, hkv = 512, 96, 1e4, 1400, 4, 2
    qb, kb, vb = make_qkv(140, 1, n, n, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    qf, kf, vf = bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(1, n, hkv), dtype=torch.uint8, device="cuda:0")
    seen = []
    for lo, hi in ((0, 300), (300, 513), (513, 700), (700, 1025), (1025, 1400)):
        qc = q[:, lo:hi].contiguous()
        kc, vc = k[:, :hi].contiguous(), v[:, :hi].contiguous()
        ref = oracle.bifocal_three_pass(qf[:, lo:hi], kf[:, :hi], vf[:, :hi], big_l, w, base)
        seen.append(ref["g"])
        for form in ("fused", "ws"):
            out = torch.empty_like(qc)
            lse = torch.empty((1, hq, hi - lo), dtype=torch.float32, device="cuda:0")
            print(f"chunk [{lo}, {hi}) g={ref['g']} form={form}", flush=True)
            if form == "fused":
                jl.jl_bifocal_prefill(qc, kc, vc, out, lse, big_l, w, base)
            else:
                jl.jl_bifocal_prefill_ws(qc, kc, vc, out, lse, big_l, w, base, ws)
            torch.cuda.synchronize()
            assert_parity(to_f64(out), ref["out"], f"chunk [{lo}, {hi}) {form}")
            assert_parity(lse.cpu().numpy().astype(np.float64), ref["lse"], "lse", max_tol=lse_tol(ref["g"]),
                          mean_tol=LSE_MEAN_TOL)
    assert seen == [1, 2, 2, 3, 3]
