"""A seeded sweep of random small shapes through every prefill and decode entry
point, each against the fp64 oracle (parity bar as everywhere: max-abs 1e-2,
mean-abs 1e-3).  The shapes draw batch, lengths, GQA group, windows, RoPE base and
schedule at random, so that combinations no hand-picked case covers (ragged
tails against every window, factors well above 4, chunks of any size) are run.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, normal_bf16

from gpu_helpers import LSE_MEAN_TOL, LSE_TOL, assert_parity, to_device, to_f64

pytestmark = pytest.mark.gpu

N_CASES = 32


def _draw(seed):
    rng = np.random.default_rng(10_000 + seed)
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    n_kv = int(rng.integers(2, 1500))
    n_q = int(rng.integers(1, n_kv + 1))
    big_l = int(rng.integers(2, max(3, n_kv)))
    w = int(rng.integers(1, big_l))             # W < L so that every schedule applies
    base = float(rng.choice([1e4, 5e5, 1e6]))
    schedule = str(rng.choice(list(oracle.SCHEDULES)))
    b = int(rng.integers(1, 3))
    return dict(b=b, hq=hq, hkv=hkv, n_kv=n_kv, n_q=n_q, big_l=big_l, w=w, base=base, schedule=schedule)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_prefill(seed):
    c = _draw(seed)
    print(f"random prefill case {seed}: {c}", flush=True)
    b, hq, hkv, n_kv, n_q = c["b"], c["hq"], c["hkv"], c["n_kv"], c["n_q"]
    qb = normal_bf16(900 + seed, 0, (b, n_q, hq, 128))
    kb = normal_bf16(900 + seed, 1, (b, n_kv, hkv, 128))
    vb = normal_bf16(900 + seed, 2, (b, n_kv, hkv, 128))
    q, k, v = to_device(qb), to_device(kb), to_device(vb)
    ref = oracle.bifocal_three_pass(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb), c["big_l"],
                                    c["w"], c["base"], schedule=c["schedule"])
    ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(b, n_kv, hkv), dtype=torch.uint8, device="cuda:0")
    for form in ("two_launch", "single_kernel", "positions"):
        out = torch.empty_like(q)
        lse = torch.empty((b, hq, n_q), dtype=torch.float32, device="cuda:0")
        if form == "two_launch":
            jl.jl_bifocal_prefill_sched(q, k, v, out, lse, c["big_l"], c["w"], c["base"], c["schedule"], ws)
        elif form == "single_kernel":
            jl.jl_bifocal_prefill_sched(q, k, v, out, lse, c["big_l"], c["w"], c["base"], c["schedule"], None)
        else:
            qp = torch.arange(n_kv - n_q, n_kv, dtype=torch.int32, device="cuda:0")
            jl.jl_bifocal_prefill_positions(q, k, v, out, lse, qp, c["big_l"], c["w"], c["base"], ws,
                                            schedule=c["schedule"])
        torch.cuda.synchronize()
        assert_parity(to_f64(out), ref["out"], f"{form} out")
        assert_parity(lse.cpu().numpy().astype(np.float64), ref["lse"], f"{form} lse", max_tol=LSE_TOL,
                      mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_varlen_prefill_and_decode(seed):
    c = _draw(seed)
    rng = np.random.default_rng(20_000 + seed)
    nb = int(rng.integers(1, 5))
    lens = [int(rng.integers(1, 1500)) for _ in range(nb)]
    chunks = [int(rng.integers(0, s + 1)) for s in lens]
    print(f"random varlen case {seed}: {c} lens={lens} chunks={chunks}", flush=True)
    hq, hkv, n_max = c["hq"], c["hkv"], max(lens)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    total = max(int(cu[-1]), 1)
    qb = normal_bf16(950 + seed, 0, (total, hq, 128))
    kb = normal_bf16(950 + seed, 1, (nb, n_max, hkv, 128))
    vb = normal_bf16(950 + seed, 2, (nb, n_max, hkv, 128))
    for bi, s in enumerate(lens):
        kb[bi, s:] = np.uint16(0x7FC0)
        vb[bi, s:] = np.uint16(0x7FC0)
    q, kc, vc = to_device(qb), to_device(kb), to_device(vb)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    kf, vf = bf16_bits_to_f64(kb), bf16_bits_to_f64(vb)
    if cu[-1] > 0:
        out = torch.empty_like(q)
        lse = torch.empty((hq, total), dtype=torch.float32, device="cuda:0")
        ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(nb, n_max, hkv), dtype=torch.uint8, device="cuda:0")
        jl.jl_bifocal_prefill_varlen(q, kc, vc, out, lse, torch.tensor(cu, device="cuda:0"), sl, max(chunks),
                                     c["big_l"], c["w"], c["base"], ws, schedule=c["schedule"])
        torch.cuda.synchronize()
        ro, rl = oracle.bifocal_prefill_varlen(bf16_bits_to_f64(qb), cu, kf, vf, lens, c["big_l"], c["w"], c["base"],
                                               schedule=c["schedule"])
        assert_parity(to_f64(out), ro, "varlen prefill out")
        assert_parity(lse.cpu().numpy().astype(np.float64), rl, "varlen prefill lse", max_tol=LSE_TOL,
                      mean_tol=LSE_MEAN_TOL)
    # decode: one new token per sequence (query at s_b - 1)
    qd_b = normal_bf16(970 + seed, 0, (nb, 1, hq, 128))
    qd = to_device(qd_b)
    od = torch.empty_like(qd)
    ld = torch.empty((nb, hq, 1), dtype=torch.float32, device="cuda:0")
    wsd = torch.empty(jl.jl_bifocal_decode_workspace_size(nb, n_max, hq, hkv), dtype=torch.uint8, device="cuda:0")
    jl.jl_bifocal_decode_sched(qd, kc, vc, od, ld, sl, c["big_l"], c["w"], c["base"], c["schedule"], wsd)
    torch.cuda.synchronize()
    q64 = bf16_bits_to_f64(qd_b)
    for bi, s in enumerate(lens):
        o, l = oracle.bifocal_decode(q64[bi:bi + 1], kf[bi:bi + 1, :s], vf[bi:bi + 1, :s], c["big_l"], c["w"],
                                     c["base"], schedule=c["schedule"])
        assert_parity(to_f64(od[bi:bi + 1]), o, f"decode seq {bi} out")
        assert_parity(ld[bi:bi + 1].cpu().numpy().astype(np.float64), l, f"decode seq {bi} lse", max_tol=LSE_TOL,
                      mean_tol=LSE_MEAN_TOL)
