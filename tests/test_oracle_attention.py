"""Pins for the oracle's attention functions (CPU only).

The three-pass inclusion-exclusion form (O1) and the brute-force per-pair
selection form (O2) are two different formulations of the same definition
(ResearchPod summary, 2nd paragraph; ResearchPod transcript, cache and prefill
exchanges; Abstract).  They are checked against each other, against torch's
fp64 scaled_dot_product_attention where the method must reduce to the base
model (Abstract: exact recovery at short inputs), against a hand-derived closed
form at D = 2, and against properties that hold for any input.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.bifocal as ob
from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64, make_qkv

# Parity bar of the GPU tests (bf16 in, fp32 accumulate): used here to show the
# bar separates the right definition from plausible off-by-one variants.
MAX_ABS_TOL = 1e-2
MEAN_ABS_TOL = 1e-3


def _raw_inputs(seed, b, n_q, n_kv, hq, hkv, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, n_q, hq, d))
    k = rng.standard_normal((b, n_kv, hkv, d))
    v = rng.standard_normal((b, n_kv, hkv, d))
    return q, k, v


def _prerotate(q_raw, k_raw, base):
    """Cached vectors: rotated at their original positions."""
    n_q, n_kv, d = q_raw.shape[1], k_raw.shape[1], q_raw.shape[-1]
    th = oracle.rope_frequencies(d, base)
    qp = oracle.query_positions(n_q, n_kv).astype(np.float64)
    kp = np.arange(n_kv, dtype=np.float64)
    q = oracle.rotate_half_pairs(q_raw, (qp[:, None] * th)[None, :, None, :])
    k = oracle.rotate_half_pairs(k_raw, (kp[:, None] * th)[None, :, None, :])
    return q, k


def _tiny_grid():
    cases = []
    # (s, n_q, L, W, D, hq, hkv, base)
    for s, big_l, w in [(1, 1, 1), (2, 1, 1), (3, 2, 1), (7, 2, 2), (7, 4, 4), (16, 4, 2), (16, 8, 8),
                        (17, 8, 4), (33, 16, 8), (33, 32, 1), (64, 16, 8), (64, 32, 32), (65, 32, 8),
                        (100, 16, 4), (100, 32, 8), (128, 32, 8), (128, 16, 16), (97, 8, 8)]:
        cases.append((s, s, big_l, w, 8, 1, 1, 1e4))
    cases += [
        (64, 64, 16, 4, 16, 4, 2, 1e6),
        (64, 5, 16, 4, 16, 4, 2, 1e4),       # queries are the last 5 positions
        (33, 1, 8, 2, 16, 2, 1, 1e4),        # decode-shaped
        (48, 48, 16, 16, 128, 1, 1, 1e6),    # W == L, full head size
        (40, 40, 8, 4, 128, 2, 2, 1e4),
    ]
    return cases


@pytest.mark.parametrize("s,n_q,big_l,w,d,hq,hkv,base", _tiny_grid())
def test_three_pass_equals_bruteforce(s, n_q, big_l, w, d, hq, hkv, base):
    q_raw, k_raw, v = _raw_inputs(s * 1000 + d, 1, n_q, s, hq, hkv, d)
    q, k = _prerotate(q_raw, k_raw, base)
    r = oracle.bifocal_three_pass(q, k, v, big_l, w, base)
    o2, lse2 = oracle.bifocal_bruteforce(q_raw, k_raw, v, big_l, w, base)
    assert r["g"] == oracle.group_factor(s, big_l)
    assert np.abs(r["out"] - o2).max() <= 1e-12 * max(1.0, np.abs(v).max())
    assert np.abs(r["lse"] - lse2).max() <= 1e-11


def test_two_dim_closed_form():
    # D = 2 -> one rotate-half pair with theta_0 = 1: position P turns a vector by P
    # radians.  s = 5, L = 2 -> g = 3; W = 2.  Expected (P_q, P_k) per causal pair,
    # worked out by hand from the local/remote rule (local iff p - j <= W - 1,
    # otherwise both positions divided by g):
    sel = {
        (0, 0): (0, 0),
        (1, 0): (1, 0), (1, 1): (1, 1),
        (2, 0): (0, 0), (2, 1): (2, 1), (2, 2): (2, 2),
        (3, 0): (1, 0), (3, 1): (1, 0), (3, 2): (3, 2), (3, 3): (3, 3),
        (4, 0): (1, 0), (4, 1): (1, 0), (4, 2): (1, 0), (4, 3): (4, 3), (4, 4): (4, 4),
    }
    rng = np.random.default_rng(11)
    s = 5
    r_q, a_q = rng.uniform(0.5, 2.0, s), rng.uniform(-3, 3, s)
    r_k, a_k = rng.uniform(0.5, 2.0, s), rng.uniform(-3, 3, s)
    v = rng.standard_normal((1, s, 1, 3))
    tau = 1.0 / math.sqrt(2.0)
    expected = np.zeros((s, 3))
    for p in range(s):
        sc = np.array([tau * r_q[p] * r_k[j] * math.cos((a_q[p] + sel[p, j][0]) - (a_k[j] + sel[p, j][1]))
                       for j in range(p + 1)])
        e = np.exp(sc - sc.max())
        expected[p] = (e / e.sum()) @ v[0, :p + 1, 0]
    # cached vectors, rotated at original positions, in polar form
    q = np.array([[r_q[p] * math.cos(a_q[p] + p), r_q[p] * math.sin(a_q[p] + p)] for p in range(s)])
    k = np.array([[r_k[j] * math.cos(a_k[j] + j), r_k[j] * math.sin(a_k[j] + j)] for j in range(s)])
    raw_q = np.array([[r_q[p] * math.cos(a_q[p]), r_q[p] * math.sin(a_q[p])] for p in range(s)])
    raw_k = np.array([[r_k[j] * math.cos(a_k[j]), r_k[j] * math.sin(a_k[j])] for j in range(s)])
    # The oracles take V with the head size of q and k (2 here): check one V column
    # at a time, copied into both slots.
    for col in range(3):
        vv = np.repeat(v[..., col:col + 1], 2, axis=-1)
        r = oracle.bifocal_three_pass(q[None, :, None], k[None, :, None], vv, 2, 2, 1e4)
        assert r["g"] == 3
        assert np.allclose(r["out"][0, :, 0, 0], expected[:, col], atol=1e-12)
        o2, _ = oracle.bifocal_bruteforce(raw_q[None, :, None], raw_k[None, :, None], vv, 2, 2, 1e4)
        assert np.allclose(o2[0, :, 0, 0], expected[:, col], atol=1e-12)


@pytest.mark.parametrize("s,big_l,w", [(40, 8, 4), (64, 16, 1), (31, 31, 31), (50, 1, 1)])
def test_value_ones_gives_ones(s, big_l, w):
    q, k, _ = _raw_inputs(5, 1, s, s, 2, 1, 16)
    v = np.ones((1, s, 1, 16))
    r = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e4)
    assert np.abs(r["out"] - 1.0).max() < 1e-12


def test_value_identity_gives_probabilities():
    s, d, big_l, w = 24, 32, 6, 3
    q_raw, k_raw, _ = _raw_inputs(6, 1, s, s, 1, 1, d)
    v = np.zeros((1, s, 1, d))
    v[0, np.arange(s), 0, np.arange(s)] = 1.0
    q, k = _prerotate(q_raw, k_raw, 1e4)
    probs = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e4)["out"][0, :, 0, :s]
    assert np.allclose(probs.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(probs >= -1e-12)
    assert np.all(np.triu(probs, 1) == 0.0)          # nothing after the query
    o2, _ = oracle.bifocal_bruteforce(q_raw, k_raw, v, big_l, w, 1e4)
    assert np.allclose(probs, o2[0, :, 0, :s], atol=1e-12)


def _torch_causal(q, k, v, scale):
    """torch fp64 SDPA with an explicit bottom-right causal mask and GQA expansion."""
    b, n_q, hq, d = q.shape
    n_kv, hkv = k.shape[1], k.shape[2]
    rep = hq // hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(rep, dim=1)
    pos = torch.arange(n_kv - n_q, n_kv)[:, None]
    mask = torch.arange(n_kv)[None, :] <= pos
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("s,n_q,big_l,w,hq,hkv", [(64, 64, 64, 8, 2, 1), (100, 30, 128, 128, 4, 2),
                                                  (512, 512, 512, 128, 1, 1), (200, 1, 256, 16, 4, 1)])
def test_short_inputs_recover_base_model(s, n_q, big_l, w, hq, hkv):
    # s <= L -> g = 1: every rotation is the original one and the merge must give
    # plain causal attention (Abstract: the base model is recovered exactly).
    q, k, v = _raw_inputs(7, 2, n_q, s, hq, hkv, 64)
    r = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e6)
    assert r["g"] == 1
    ref = _torch_causal(q, k, v, 1.0 / 8.0)
    assert np.abs(r["out"] - ref).max() < 1e-12
    plain, plain_lse = oracle.plain_causal_attention(q, k, v)
    assert np.abs(plain - ref).max() < 1e-12
    assert np.abs(r["lse"] - plain_lse).max() < 1e-12


def test_rows_without_remote_keys_equal_plain():
    s, big_l, w = 256, 64, 32                      # g = 4
    q, k, v = _raw_inputs(8, 1, s, s, 2, 1, 32)
    r = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e4)
    plain, _ = oracle.plain_causal_attention(q, k, v)
    assert r["g"] == 4
    assert np.abs(r["out"][:, :w] - plain[:, :w]).max() < 1e-12
    assert np.abs(r["out"][:, w:] - plain[:, w:]).max() > 1e-3   # and the others differ


def test_causality_bitwise():
    s, big_l, w = 96, 16, 8
    q, k, v = _raw_inputs(9, 1, s, s, 1, 1, 16)
    base = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e4, row_block=8)["out"]
    k2, v2 = k.copy(), v.copy()
    cut = 40
    k2[:, cut + 1:] += 3.0
    v2[:, cut + 1:] *= -2.0
    pert = oracle.bifocal_three_pass(q, k2, v2, big_l, w, 1e4, row_block=8)["out"]
    assert np.array_equal(base[:, :cut + 1], pert[:, :cut + 1])


def test_decode_equals_last_prefill_row():
    s, big_l, w = 300, 64, 16
    q, k, v = _raw_inputs(10, 1, s, s, 4, 2, 32)
    full = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e6)
    o, lse = oracle.bifocal_decode(q[:, -1:], k, v, big_l, w, 1e6)
    assert np.abs(o[:, 0] - full["out"][:, -1]).max() < 1e-12
    assert np.abs(lse[..., 0] - full["lse"][..., -1]).max() < 1e-12


def test_row_subset_matches_full():
    s, big_l, w = 200, 32, 8
    q, k, v = _raw_inputs(12, 1, s, s, 2, 2, 16)
    full = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e4)
    rows = np.array([0, 7, 8, 31, 32, 33, 100, 199])
    sub = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e4, rows=rows)
    assert np.abs(sub["out"] - full["out"][:, rows]).max() < 1e-12
    assert np.abs(sub["lse"] - full["lse"][:, :, rows]).max() < 1e-12


def _fails_bar(a, b, margin):
    d = np.abs(a - b)
    return d.max() > margin * MAX_ABS_TOL or d.mean() > margin * MEAN_ABS_TOL


@pytest.mark.parametrize("q_scale", [1.0, 4.0])
def test_parity_bar_detects_off_by_one(monkeypatch, q_scale):
    # Causal prefill, 1 head, D 128, s 2048, L 512, W 128 (g = 4): the parity bar
    # must reject g +- 1 and W +- 1 by a wide margin, or an off-by-one in the
    # kernels could pass it.
    q, k, v = [bf16_bits_to_f64(x) for x in make_qkv(0, 1, 2048, 2048, 1, 1, 128, q_scale=q_scale)]
    ref = oracle.bifocal_three_pass(q, k, v, 512, 128, 1e4)
    assert ref["g"] == 4
    for w in (127, 129):
        assert _fails_bar(oracle.bifocal_three_pass(q, k, v, 512, w, 1e4)["out"], ref["out"], 5)
    orig = ob.group_factor
    for dg in (-1, 1):
        monkeypatch.setattr(ob, "group_factor", lambda s, big_l, dg=dg: orig(s, big_l) + dg)
        assert _fails_bar(oracle.bifocal_three_pass(q, k, v, 512, 128, 1e4)["out"], ref["out"], 5)


def test_parity_bar_detects_seam_shift():
    # A Self-Extend-style seam shift (query aliased to p//g + W - W//g) is a
    # different reading; the bar must tell it apart.
    s, big_l, w, d = 96, 24, 8, 16
    q_raw, k_raw, v = _raw_inputs(13, 1, s, s, 1, 1, d)
    g = oracle.group_factor(s, big_l)

    def shifted(p, j):
        if p - j <= w - 1:
            return p, j
        return p // g + w - w // g, j // g

    right, _ = oracle.bifocal_bruteforce(q_raw * 2, k_raw, v, big_l, w, 1e4)
    wrong, _ = oracle.bifocal_bruteforce(q_raw * 2, k_raw, v, big_l, w, 1e4, select=shifted)
    assert _fails_bar(wrong, right, 5)


def test_decode_varlen_equals_bruteforce_per_sequence():
    # three sequences in one padded cache: lengths 5, 17, 40 with L = 8, W = 3 give
    # g = 1, 3, 5, i.e. plain, bifocal, and bifocal with a larger factor; rows past a
    # sequence's length are NaN, so a read beyond its prefix would poison its output
    big_l, w, base, d, hq, hkv = 8, 3, 1e4, 16, 4, 2
    lens = [5, 17, 40]
    n_max = max(lens)
    rng = np.random.default_rng(4242)
    q = np.zeros((3, 1, hq, d))
    k = np.full((3, n_max, hkv, d), np.nan)
    v = np.full((3, n_max, hkv, d), np.nan)
    expect = []
    for bi, s in enumerate(lens):
        q_raw = rng.standard_normal((1, 1, hq, d))
        k_raw = rng.standard_normal((1, s, hkv, d))
        v_s = rng.standard_normal((1, s, hkv, d))
        q_rot, k_rot = _prerotate(q_raw, k_raw, base)
        q[bi], k[bi, :s], v[bi, :s] = q_rot[0], k_rot[0], v_s[0]
        expect.append(oracle.bifocal_bruteforce(q_raw, k_raw, v_s, big_l, w, base))
    out, lse = oracle.bifocal_decode_varlen(q, k, v, lens, big_l, w, base)
    assert [oracle.group_factor(s, big_l) for s in lens] == [1, 3, 5]
    for bi in range(3):
        o2, l2 = expect[bi]
        assert np.abs(out[bi:bi + 1] - o2).max() <= 1e-12 * np.nanmax(np.abs(v))
        assert np.abs(lse[bi:bi + 1] - l2).max() <= 1e-11
    # with every length inside the pretrained window the method is the base model
    out_b, lse_b = oracle.bifocal_decode_varlen(q, k, v, lens, 64, w, base)
    out_p, lse_p = oracle.plain_decode_varlen(q, k, v, lens)
    assert np.abs(out_b - out_p).max() <= 1e-12 and np.abs(lse_b - lse_p).max() <= 1e-12
    # and plain matches torch's fp64 attention of each query over its own prefix
    for bi, s in enumerate(lens):
        qt = torch.from_numpy(q[bi:bi + 1]).permute(0, 2, 1, 3)
        kt = torch.from_numpy(np.repeat(k[bi:bi + 1, :s], hq // hkv, axis=2)).permute(0, 2, 1, 3)
        vt = torch.from_numpy(np.repeat(v[bi:bi + 1, :s], hq // hkv, axis=2)).permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).permute(0, 2, 1, 3).numpy()
        assert np.abs(out_p[bi:bi + 1] - ref).max() <= 1e-12


@pytest.mark.parametrize("n_q,n_kv,w,hq,hkv", [(40, 40, 7, 4, 2), (9, 50, 16, 2, 1), (1, 33, 5, 4, 4), (64, 64, 1, 2, 2)])
def test_sliding_window_attention_pins(n_q, n_kv, w, hq, hkv):
    q, k, v = _raw_inputs(7000 + n_kv * 10 + w, 2, n_q, n_kv, hq, hkv, 16)
    out, lse = oracle.sliding_window_attention(q, k, v, w)
    # torch's fp64 attention with an explicit band mask (query i at position n_kv - n_q + i)
    pos = np.arange(n_kv - n_q, n_kv)
    dist = pos[:, None] - np.arange(n_kv)[None, :]
    band = torch.from_numpy((dist >= 0) & (dist <= w - 1))
    rep = hq // hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.repeat(k, rep, axis=2)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.repeat(v, rep, axis=2)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=band).permute(0, 2, 1, 3).numpy()
    assert np.abs(out - ref).max() <= 1e-12
    # it is the local view (pass A) of the three-pass form, for any L >= W
    r = oracle.bifocal_three_pass(q, k, v, max(w, 4), w, 1e4)
    o_a, l_a = r["passes"]["A"]
    assert np.abs(out - o_a).max() <= 1e-12 and np.abs(lse - l_a).max() <= 1e-12
    # a window covering every key is plain causal attention
    o_p, l_p = oracle.plain_causal_attention(q, k, v)
    o_w, l_w = oracle.sliding_window_attention(q, k, v, n_kv)
    assert np.abs(o_w - o_p).max() <= 1e-12 and np.abs(l_w - l_p).max() <= 1e-12
    if w == 1:   # only the query's own key: the output is that key's value
        for i, p in enumerate(pos):
            assert np.abs(out[:, i] - np.repeat(v[:, p], rep, axis=1)).max() <= 1e-15


# ---------------------------------------------------------------------------
# Long-range schedule variants: seam-shifted grouping and fractional scaling
# (seventnews.com, 1st section: l(s) follows the current length; the pages also
# speak of realigning the two branches at the seam).  The pages print no value
# for either variant, so these pins check the two formulations against each
# other and against what the definitions fix.

def _schedule_grid():
    # (s, n_q, L, W, D, hq, hkv, base); seam needs W < L, fractional L >= 2
    return [(7, 7, 3, 2, 8, 1, 1, 1e4), (16, 16, 4, 2, 8, 1, 1, 1e4), (33, 33, 16, 8, 8, 1, 1, 1e4),
            (64, 64, 16, 4, 16, 4, 2, 1e6), (100, 100, 32, 8, 8, 1, 1, 1e4), (65, 9, 16, 15, 16, 2, 1, 1e4),
            (40, 1, 8, 3, 128, 2, 2, 1e4), (128, 128, 9, 8, 8, 1, 1, 1e4)]


@pytest.mark.parametrize("schedule", ["seam", "fractional"])
@pytest.mark.parametrize("s,n_q,big_l,w,d,hq,hkv,base", _schedule_grid())
def test_schedule_three_pass_equals_bruteforce(schedule, s, n_q, big_l, w, d, hq, hkv, base):
    q_raw, k_raw, v = _raw_inputs(s * 77 + w, 1, n_q, s, hq, hkv, d)
    q, k = _prerotate(q_raw, k_raw, base)
    r = oracle.bifocal_three_pass(q, k, v, big_l, w, base, schedule=schedule)
    o2, lse2 = oracle.bifocal_bruteforce(q_raw, k_raw, v, big_l, w, base, schedule=schedule)
    assert np.abs(r["out"] - o2).max() <= 1e-12 * max(1.0, np.abs(v).max())
    assert np.abs(r["lse"] - lse2).max() <= 1e-11
    # and the variant is a different attention from the integer grouping once s > L
    base_out = oracle.bifocal_three_pass(q, k, v, big_l, w, base)["out"]
    assert np.abs(r["out"] - base_out).max() > 1e-6


@pytest.mark.parametrize("schedule", list(oracle.SCHEDULES))
@pytest.mark.parametrize("s,big_l,w", [(40, 40, 8), (33, 64, 4), (16, 17, 16)])
def test_schedules_recover_base_model(schedule, s, big_l, w):
    # s <= L: every schedule leaves the positions alone (g = 1, no shift; l = 1)
    q, k, v = _raw_inputs(5 * s + w, 2, s, s, 4, 2, 16)
    r = oracle.bifocal_three_pass(q, k, v, big_l, w, 1e4, schedule=schedule)
    o_p, l_p = oracle.plain_causal_attention(q, k, v)
    assert r["g"] == 1
    assert np.abs(o_p - _torch_causal(q, k, v, 0.25)).max() < 1e-12
    assert np.abs(r["out"] - o_p).max() <= 1e-12 and np.abs(r["lse"] - l_p).max() <= 1e-12


@pytest.mark.parametrize("s,big_l,w", [(s, big_l, w) for s in (1, 2, 9, 50, 257, 1000)
                                       for big_l in (2, 3, 8, 33) for w in (1, 2, 7, 32) if w < big_l])
def test_seam_factor_minimal_over_all_pairs(s, big_l, w):
    # brute force over every remote (query, key) pair of a length-s input: the
    # largest shifted distance fits in the window for g, and not for g - 1
    def max_remote_distance(g):
        shift = w - w // g
        return max((p // g + shift - j // g for p in range(s) for j in range(0, p - w + 1)), default=0)

    g, a_q, a_k = oracle.long_range_schedule(s, big_l, w, "seam")
    assert g == oracle.seam_group_factor(s, big_l, w)
    p = np.arange(s)
    remote = [(pp, j) for pp in range(s) for j in range(0, pp - w + 1)]
    if remote:
        pq = np.array([r[0] for r in remote])
        pk = np.array([r[1] for r in remote])
        assert (a_q(pq) - a_k(pk)).max() == max_remote_distance(g) <= big_l - 1
    assert np.array_equal(a_k(p), p // g)
    if g > 1 and s > w:
        assert max_remote_distance(g - 1) > big_l - 1


# g worked out by hand: e.g. s = 40, L = 8, W = 5 needs floor(39/g) - floor(5/g) <= 2,
# which g = 13 misses (3) and g = 14 meets; at the 128K workload g goes 4 -> 5.
@pytest.mark.parametrize("s,big_l,w,g_expect", [(40, 8, 5, 14), (200, 16, 5, 19), (1000, 64, 16, 21),
                                                (131072, 32768, 4096, 5), (131072, 32768, 1, 5)])
def test_seam_distances_continue_the_window(s, big_l, w, g_expect):
    # p - j = W (the first remote key): the shifted distance is W or W + 1, so it
    # continues the local distances 0..W-1; the unshifted grouping gives about W / g
    g, a_q, a_k = oracle.long_range_schedule(s, big_l, w, "seam")
    assert g == g_expect
    j = np.arange(0, s - w)
    dists = set((a_q(j + w) - a_k(j)).tolist())
    assert dists <= {w, w + 1} and w in dists
    # deeper remote keys are farther: distance never decreases as j moves back
    d_all = a_q(np.full(s - w, s - 1)) - a_k(np.arange(s - w))
    assert np.all(np.diff(d_all) <= 0)
    if g > 1 and w >= g:
        g0, aq0, ak0 = oracle.long_range_schedule(s, big_l, w, "grouped")
        assert (aq0(j + w) - ak0(j)).max() <= w // g0 + 1 < w


def test_fractional_two_dim_closed_form():
    # D = 2: one rotate-half pair with theta_0 = 1.  s = 7, L = 3 -> l = 3; W = 2.
    # Remote pairs see the positions p / l and j / l, local pairs p and j.
    rng = np.random.default_rng(12)
    s, big_l, w = 7, 3, 2
    lf = oracle.fractional_factor(s, big_l)
    assert lf == 3.0
    r_q, a_q = rng.uniform(0.5, 2.0, s), rng.uniform(-3, 3, s)
    r_k, a_k = rng.uniform(0.5, 2.0, s), rng.uniform(-3, 3, s)
    v = rng.standard_normal((1, s, 1, 2))
    tau = 1.0 / math.sqrt(2.0)
    expected = np.zeros((s, 2))
    for p in range(s):
        sc = []
        for j in range(p + 1):
            pq, pk = (p, j) if p - j <= w - 1 else (p / 3.0, j / 3.0)
            sc.append(tau * r_q[p] * r_k[j] * math.cos((a_q[p] + pq) - (a_k[j] + pk)))
        sc = np.array(sc)
        e = np.exp(sc - sc.max())
        expected[p] = (e / e.sum()) @ v[0, :p + 1, 0]
    q = np.array([[r_q[p] * math.cos(a_q[p] + p), r_q[p] * math.sin(a_q[p] + p)] for p in range(s)])
    k = np.array([[r_k[j] * math.cos(a_k[j] + j), r_k[j] * math.sin(a_k[j] + j)] for j in range(s)])
    r = oracle.bifocal_three_pass(q[None, :, None], k[None, :, None], v, big_l, w, 1e4, schedule="fractional")
    assert np.abs(r["out"][0, :, 0] - expected).max() <= 1e-12


def test_prefill_varlen_equals_bruteforce_per_sequence():
    # four sequences in one padded cache: (new rows, keys) = (20, 20), (7, 33), (0, 9),
    # (1, 40) with L = 8, W = 3; rows past a prefix are NaN
    big_l, w, base, d, hq, hkv = 8, 3, 1e4, 16, 4, 2
    spec = [(20, 20), (7, 33), (0, 9), (1, 40)]
    n_max = max(s for _, s in spec)
    rng = np.random.default_rng(777)
    cu = np.concatenate([[0], np.cumsum([n for n, _ in spec])])
    q = np.zeros((cu[-1], hq, d))
    k = np.full((len(spec), n_max, hkv, d), np.nan)
    v = np.full((len(spec), n_max, hkv, d), np.nan)
    raws = []
    for bi, (n, s) in enumerate(spec):
        q_raw = rng.standard_normal((1, n, hq, d))
        k_raw = rng.standard_normal((1, s, hkv, d))
        v_s = rng.standard_normal((1, s, hkv, d))
        q_rot, k_rot = _prerotate(q_raw, k_raw, base)
        q[cu[bi]:cu[bi + 1]], k[bi, :s], v[bi, :s] = q_rot[0], k_rot[0], v_s[0]
        raws.append((q_raw, k_raw, v_s))
    for sched in oracle.SCHEDULES:
        out, lse = oracle.bifocal_prefill_varlen(q, cu, k, v, [s for _, s in spec], big_l, w, base, schedule=sched)
        for bi, (n, s) in enumerate(spec):
            if n == 0:
                continue
            o2, l2 = oracle.bifocal_bruteforce(*raws[bi], big_l, w, base, schedule=sched)
            assert np.abs(out[cu[bi]:cu[bi + 1]] - o2[0]).max() <= 1e-12
            assert np.abs(lse[:, cu[bi]:cu[bi + 1]] - l2[0]).max() <= 1e-11
    # plain: torch's fp64 attention per sequence
    out_p, _ = oracle.bifocal_prefill_varlen(q, cu, k, v, [s for _, s in spec], big_l, w, base, bifocal=False)
    for bi, (n, s) in enumerate(spec):
        if n == 0:
            continue
        qt = torch.from_numpy(q[cu[bi]:cu[bi + 1]][None]).permute(0, 2, 1, 3)
        kt = torch.from_numpy(np.repeat(k[bi:bi + 1, :s], hq // hkv, axis=2)).permute(0, 2, 1, 3)
        vt = torch.from_numpy(np.repeat(v[bi:bi + 1, :s], hq // hkv, axis=2)).permute(0, 2, 1, 3)
        mask = torch.from_numpy(np.arange(s)[None, :] <= (s - n + np.arange(n))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask).permute(0, 2, 1, 3)
        assert np.abs(out_p[cu[bi]:cu[bi + 1]] - ref.numpy()[0]).max() <= 1e-12


@pytest.mark.parametrize("schedule", list(oracle.SCHEDULES))
def test_explicit_positions_are_rows_of_the_whole_prefill(schedule):
    # queries at a sorted subset of positions (gaps, repeats) of a 90-key context
    s, big_l, w, d, hq, hkv, base = 90, 16, 5, 16, 4, 2, 1e4
    rng = np.random.default_rng(90)
    pos = np.sort(rng.choice(s, 23, replace=True))
    q_raw, k_raw, v = _raw_inputs(91, 1, s, s, hq, hkv, d)
    q_all, k = _prerotate(q_raw, k_raw, base)
    full = oracle.bifocal_three_pass(q_all, k, v, big_l, w, base, schedule=schedule)
    r = oracle.bifocal_three_pass(q_all[:, pos], k, v, big_l, w, base, schedule=schedule, positions=pos)
    assert np.abs(r["out"] - full["out"][:, pos]).max() <= 1e-12
    assert np.abs(r["lse"] - full["lse"][:, :, pos]).max() <= 1e-12
    o2, l2 = oracle.bifocal_bruteforce(q_raw[:, pos], k_raw, v, big_l, w, base, schedule=schedule, positions=pos)
    assert np.abs(r["out"] - o2).max() <= 1e-12 and np.abs(r["lse"] - l2).max() <= 1e-11
    if schedule == "grouped":
        op, lp = oracle.plain_causal_attention(q_all[:, pos], k, v, positions=pos)
        mask = torch.from_numpy(np.arange(s)[None, :] <= pos[:, None])
        rep = hq // hkv
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q_all[:, pos]).permute(0, 2, 1, 3),
            torch.from_numpy(np.repeat(k, rep, axis=2)).permute(0, 2, 1, 3),
            torch.from_numpy(np.repeat(v, rep, axis=2)).permute(0, 2, 1, 3), attn_mask=mask).permute(0, 2, 1, 3)
        assert np.abs(op - ref.numpy()).max() <= 1e-12
    with pytest.raises(ValueError):
        oracle.query_positions(3, 10, [0, 4, 10])


def test_paged_decode_equals_contiguous():
    # a contiguous cache scattered row by row into shuffled pages of 8 positions,
    # every unused page NaN: gathering recovers it, and the paged decode is the
    # variable-length decode on the contiguous cache
    big_l, w, base, d, hq, hkv, ps = 8, 3, 1e4, 16, 4, 2, 8
    lens = [5, 17, 40]
    n_max = 40
    pages_per_seq = n_max // ps
    rng = np.random.default_rng(55)
    k = np.full((3, n_max, hkv, d), np.nan)
    v = np.full((3, n_max, hkv, d), np.nan)
    for bi, s in enumerate(lens):
        k[bi, :s] = rng.standard_normal((s, hkv, d))
        v[bi, :s] = rng.standard_normal((s, hkv, d))
    q = rng.standard_normal((3, 1, hq, d))
    n_pages = 3 * pages_per_seq + 4
    perm = rng.permutation(n_pages)
    table = perm[:3 * pages_per_seq].reshape(3, pages_per_seq)
    kp = np.full((n_pages, ps, hkv, d), np.nan)
    vp = np.full((n_pages, ps, hkv, d), np.nan)
    for bi, s in enumerate(lens):
        for j in range(s):
            kp[table[bi, j // ps], j % ps] = k[bi, j]
            vp[table[bi, j // ps], j % ps] = v[bi, j]
    kg = oracle.gather_pages(kp, table, lens)
    for bi, s in enumerate(lens):
        assert np.array_equal(kg[bi, :s], k[bi, :s]) and np.all(np.isnan(kg[bi, s:]))
    for sched in oracle.SCHEDULES:
        o1, l1 = oracle.bifocal_decode_paged(q, kp, vp, table, lens, big_l, w, base, schedule=sched)
        if sched == "grouped":
            o2, l2 = oracle.bifocal_decode_varlen(q, k, v, lens, big_l, w, base)
            assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
        for bi, s in enumerate(lens):
            o3, l3 = oracle.bifocal_decode(q[bi:bi + 1], k[bi:bi + 1, :s], v[bi:bi + 1, :s], big_l, w, base,
                                           schedule=sched)
            assert np.array_equal(o1[bi:bi + 1], o3) and np.array_equal(l1[bi:bi + 1], l3)
    op, lp = oracle.bifocal_decode_paged(q, kp, vp, table, lens, big_l, w, base, bifocal=False)
    o4, l4 = oracle.plain_decode_varlen(q, k, v, lens)
    assert np.array_equal(op, o4) and np.array_equal(lp, l4)
