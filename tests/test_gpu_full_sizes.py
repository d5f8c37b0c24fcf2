"""GPU parity at the full workload sizes, on sampled rows.

Rows are independent, so the oracle computes a sample of rows exactly while the
GPU runs the whole problem in the launch configuration the bench times.  The
sample holds runs of 16 consecutive rows in five query blocks (the first rows,
the rows around p = W where remote keys appear, around p = L, the middle and
the last rows) plus rows next to multiples of g, over every KV head (so every
workgroup-to-head mapping of the grid is checked), for both prefill forms.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv

from gpu_helpers import LSE_MEAN_TOL, assert_parity, lse_tol, sample_rows, to_device, to_f64

pytestmark = pytest.mark.gpu

# workload id, seq, Hq, Hkv, L, W, base
FULL = {
    "qwen3_1p7b_64k": (1, 65536, 16, 8, 32768, 4096, 1e6),
    "qwen3_8b_128k": (2, 131072, 32, 8, 32768, 4096, 1e6),
    "sweep_48k": (4, 49152, 32, 8, 32768, 4096, 1e6),
    "sweep_96k": (4, 98304, 32, 8, 32768, 4096, 1e6),
}


def full_rows(s, big_l, w, g):
    """Runs of 16 rows at the start, around W, around L, in the middle and at the
    end, plus the seam and random rows of sample_rows: 80 rows or more."""
    runs = [np.arange(a, a + 16) for a in (0, w - 8, big_l - 8, s // 2 - 8, s - 16)]
    rows = np.concatenate(runs + [sample_rows(s, s, big_l, w, g, count=24)])
    return np.unique(np.clip(rows, 0, s - 1))


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled_rows(name):
    wid, s, hq, hkv, big_l, w, base = FULL[name]
    g = oracle.group_factor(s, big_l)
    qb, kb, vb = make_qkv(wid, 1, s, s, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    rows = full_rows(s, big_l, w, g)
    grp = hq // hkv
    kf, vf = bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    refs = []
    for kvh in range(hkv):
        heads = slice(kvh * grp, (kvh + 1) * grp)
        refs.append(oracle.bifocal_three_pass(bf16_bits_to_f64(qb[:, :, heads]), kf[:, :, kvh:kvh + 1],
                                              vf[:, :, kvh:kvh + 1], big_l, w, base, rows=rows))
        assert refs[-1]["g"] == g == jl.jl_group_factor(s, big_l)
    ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(1, s, hkv), dtype=torch.uint8, device="cuda:0")
    for form in ("fused", "two_launch"):
        print(f"full size {name}: s={s} Hq={hq} Hkv={hkv} g={g} form={form}, {len(rows)} rows x {hkv} KV heads",
              flush=True)
        out = torch.empty_like(q)
        lse = torch.empty((1, hq, s), dtype=torch.float32, device="cuda:0")
        if form == "fused":
            jl.jl_bifocal_prefill(q, k, v, out, lse, big_l, w, base)
        else:
            jl.jl_bifocal_prefill_ws(q, k, v, out, lse, big_l, w, base, ws)
        torch.cuda.synchronize()
        got = to_f64(out[:, rows])
        got_lse = lse[:, :, rows].cpu().numpy().astype(np.float64)
        for kvh in range(hkv):
            heads = slice(kvh * grp, (kvh + 1) * grp)
            assert_parity(got[:, :, heads], refs[kvh]["out"], f"{name} {form} kv head {kvh}")
            assert_parity(got_lse[:, heads], refs[kvh]["lse"], "lse", max_tol=lse_tol(g), mean_tol=LSE_MEAN_TOL)
        del out, lse


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


def test_batch_of_two_at_48k():
    # Batch offsets at a full-size shape: two sequences of 48K (32/8 heads, g = 2), so
    # that the second sequence's rows, keys and outputs sit past the first's 48K x 32
    # heads; sampled rows of both sequences over every KV head, both prefill forms.
    b, s, hq, hkv, big_l, w, base = 2, 49152, 32, 8, 32768, 4096, 1e6
    g = oracle.group_factor(s, big_l)
    qb, kb, vb = make_qkv(5, b, s, s, hq, hkv, 128)
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(w - 4, w + 4), np.arange(s - 8, s),
                                     rng.choice(s, 16, replace=False)]))
    grp = hq // hkv
    refs = []
    for kvh in range(hkv):
        heads = slice(kvh * grp, (kvh + 1) * grp)
        refs.append(oracle.bifocal_three_pass(bf16_bits_to_f64(qb[:, :, heads]), bf16_bits_to_f64(kb[:, :, kvh:kvh + 1]),
                                              bf16_bits_to_f64(vb[:, :, kvh:kvh + 1]), big_l, w, base, rows=rows))
    ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(b, s, hkv), dtype=torch.uint8, device="cuda:0")
    for form in ("fused", "two_launch"):
        print(f"batch 2 at 48K: form={form}, {len(rows)} rows x 2 sequences x {hkv} KV heads", flush=True)
        out = torch.empty_like(q)
        lse = torch.empty((b, hq, s), dtype=torch.float32, device="cuda:0")
        if form == "fused":
            jl.jl_bifocal_prefill(q, k, v, out, lse, big_l, w, base)
        else:
            jl.jl_bifocal_prefill_ws(q, k, v, out, lse, big_l, w, base, ws)
        torch.cuda.synchronize()
        got = to_f64(out[:, rows])
        got_lse = lse[:, :, rows].cpu().numpy().astype(np.float64)
        for kvh in range(hkv):
            heads = slice(kvh * grp, (kvh + 1) * grp)
            assert_parity(got[:, :, heads], refs[kvh]["out"], f"batch 2 {form} kv head {kvh}")
            assert_parity(got_lse[:, heads], refs[kvh]["lse"], "lse", max_tol=lse_tol(g), mean_tol=LSE_MEAN_TOL)
        del out, lse
