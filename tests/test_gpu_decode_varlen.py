"""GPU parity of the variable-length batched decode against the fp64 oracle.

Each sequence of a padded batch holds its own number of keys s_b and gets the
group factor of its own length (seventnews.com, the long-range factor follows
the current length), so one launch mixes plain sequences (g = 1) with bifocal
ones.  Cache rows past a sequence's length are NaN in every test: a read beyond
the prefix would poison that sequence's output.
"""

import numpy as np
import pytest
import torch

import oracle
import zero_shot_rope_attention_amd as jl
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, normal_bf16

from gpu_helpers import LSE_MEAN_TOL, LSE_TOL_PLAIN, assert_parity, lse_tol, to_device, to_f64

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)


def _inputs(seed, lens, hq, hkv, n_max=None):
    n_max = n_max or max(lens)
    b = len(lens)
    qb = normal_bf16(seed, 0, (b, 1, hq, 128))
    kb = normal_bf16(seed, 1, (b, n_max, hkv, 128))
    vb = normal_bf16(seed, 2, (b, n_max, hkv, 128))
    for bi, s in enumerate(lens):
        kb[bi, s:] = BF16_NAN
        vb[bi, s:] = BF16_NAN
    return qb, kb, vb


def _run(qb, kb, vb, lens, big_l=None, w=None, base=None, plain=False, varlen=True):
    b, _, hq, _ = qb.shape
    n_max, hkv = kb.shape[1], kb.shape[2]
    q, kc, vc = to_device(qb), to_device(kb), to_device(vb)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, 1), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(jl.jl_bifocal_decode_workspace_size(b, n_max, hq, hkv), dtype=torch.uint8, device="cuda:0")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    print(f"decode varlen lens={list(lens)} n_max={n_max} Hq={hq} Hkv={hkv} L={big_l} W={w} plain={plain} "
          f"varlen={varlen}", flush=True)
    if not varlen:
        if plain:
            jl.jl_plain_decode(q, kc, vc, out, lse, ws)
        else:
            jl.jl_bifocal_decode(q, kc, vc, out, lse, big_l, w, base, ws)
    elif plain:
        jl.jl_plain_decode_varlen(q, kc, vc, out, lse, sl, ws)
    else:
        jl.jl_bifocal_decode_varlen(q, kc, vc, out, lse, sl, big_l, w, base, ws)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def _f64_prefixes(kb, vb, lens):
    return [(bf16_bits_to_f64(kb[bi:bi + 1, :s]), bf16_bits_to_f64(vb[bi:bi + 1, :s])) for bi, s in enumerate(lens)]


def _oracle(qb, kb, vb, lens, big_l, w, base):
    q = bf16_bits_to_f64(qb)
    outs, lses = [], []
    for bi, (k, v) in enumerate(_f64_prefixes(kb, vb, lens)):
        o, l = oracle.bifocal_decode(q[bi:bi + 1], k, v, big_l, w, base)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs), np.concatenate(lses)


@pytest.mark.parametrize("lens", [(1, 700, 1537, 3000), (3000, 129, 2048, 513), (512, 513, 1024, 1025, 2500)])
def test_varlen_mixed_group_factors(lens):
    # L = 512, W = 128: g ranges over 1..6 across the batch; Hq 8 / Hkv 2
    big_l, w, base = 512, 128, 1e4
    qb, kb, vb = _inputs(300 + len(lens), list(lens), 8, 2)
    out, lse = _run(qb, kb, vb, lens, big_l, w, base)
    ro, rl = _oracle(qb, kb, vb, lens, big_l, w, base)
    # the oracle's own varlen function on the full padded arrays gives the same reference
    ro2, rl2 = oracle.bifocal_decode_varlen(bf16_bits_to_f64(qb), bf16_bits_to_f64(kb), bf16_bits_to_f64(vb),
                                            lens, big_l, w, base)
    assert np.array_equal(ro, ro2) and np.array_equal(rl, rl2)
    for bi, s in enumerate(lens):
        assert_parity(out[bi:bi + 1], ro[bi:bi + 1], f"seq {bi} s={s} g={oracle.group_factor(s, big_l)}")
        assert_parity(lse[bi:bi + 1], rl[bi:bi + 1], "lse", max_tol=lse_tol(oracle.group_factor(s, big_l)),
                      mean_tol=LSE_MEAN_TOL)


def test_varlen_plain_and_exact_recovery():
    lens = [100, 1, 2999, 640]
    qb, kb, vb = _inputs(310, lens, 8, 2)
    out_p, lse_p = _run(qb, kb, vb, lens, plain=True)
    q = bf16_bits_to_f64(qb)
    for bi, (k, v) in enumerate(_f64_prefixes(kb, vb, lens)):
        ro, rl = oracle.plain_causal_attention(q[bi:bi + 1], k, v)
        assert_parity(out_p[bi:bi + 1], ro, f"plain seq {bi}")
        assert_parity(lse_p[bi:bi + 1], rl, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)
    # every length inside the pretrained window: the bifocal call is the plain decode, bitwise
    out_b, lse_b = _run(qb, kb, vb, lens, 4096, 512, 1e6)
    assert np.array_equal(out_b, out_p) and np.array_equal(lse_b, lse_p)


def test_varlen_equal_lengths_is_the_batched_decode_bitwise():
    lens = [2600, 2600, 2600]
    qb, kb, vb = _inputs(320, lens, 16, 4)
    a = _run(qb, kb, vb, lens, 700, 200, 1e4)
    bb = _run(qb, kb, vb, lens, 700, 200, 1e4, varlen=False)
    assert np.array_equal(a[0], bb[0]) and np.array_equal(a[1], bb[1])


def test_varlen_workload_shape_across_group_steps():
    # Qwen3-8B-shaped decode heads (32 / 8, D 128, L 32768, W 4096, base 1e6); lengths on
    # both sides of L and 2L, so g = 1, 2, 2, 3 within one launch
    lens = [20000, 32769, 65536, 70001]
    qb, kb, vb = _inputs(330, lens, 32, 8)
    out, lse = _run(qb, kb, vb, lens, 32768, 4096, 1e6)
    ro, rl = _oracle(qb, kb, vb, lens, 32768, 4096, 1e6)
    for bi, s in enumerate(lens):
        assert_parity(out[bi:bi + 1], ro[bi:bi + 1], f"seq {bi} s={s} g={oracle.group_factor(s, 32768)}")
        assert_parity(lse[bi:bi + 1], rl[bi:bi + 1], "lse", max_tol=lse_tol(oracle.group_factor(s, 32768)),
                      mean_tol=LSE_MEAN_TOL)
