"""fp64 numpy oracle for Dynamic Bifocal RoPE attention (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may use this module.  It is independent of the HIP library: no shared code,
tables, constants or helpers, and it imports nothing from it.

Notation (the pages print no formulas; the readings taken are stated per function):

* ``s = n_kv`` keys, at cache index == original position ``j`` in ``[0, s)``.
* ``n_q`` queries at positions ``p_i = s - n_q + i`` (the newest tokens).
* pretrained window ``L``, local window ``W``, RoPE base ``b``, head size ``D``.
* ``theta_d = b ** (-2 d / D)`` for ``d < D/2``; rotate-half pairing ``(d, d + D/2)``.
* ``g = g(s)``; aliased position ``a(p) = p // g``; correction ``c(p) = a(p) - p``.
* Inputs ``q, k`` are already rotated at their original positions (the cache keeps
  original positions).  The corrected vectors are ``rot(x, c(p) theta)``.

Parity pins (see ``tests/test_oracle_*.py``):

* ``group_factor``: closed form, minimality/range invariants, values for every
  workload size (``tests/golden/group_factor.txt``), exhaustive small grids.
* ``rope_frequencies`` / ``rotate_half_pairs`` / ``rotation_matrix``: polar-form
  closed form at D=2, composition, norm, relative-position property.
* ``bifocal_three_pass``: equals ``bifocal_bruteforce`` (a different formulation)
  on a tiny grid; equals torch's fp64 ``scaled_dot_product_attention`` when
  ``s <= L``; hand-derived closed form at D=2; V=1 and V=I properties;
  causality; rows with no remote key equal plain rows.
* ``bifocal_bruteforce``: same pins as above (they check each other) plus the
  D=2 closed form, which uses neither.
* ``plain_causal_attention``: torch fp64 ``scaled_dot_product_attention``.
* ``positions`` (explicit query positions, any of the functions above): rows at
  given positions equal the rows of the whole prefill at those positions; the
  three-pass form equals the brute force; plain equals torch's fp64 attention
  with the matching causal mask.
* ``bifocal_decode``: it is ``bifocal_three_pass`` at one query row, pinned by the
  same tests plus the decode-equals-last-prefill-row check.
* ``long_range_schedule`` (seam-shifted and fractional variants): the three-pass
  form equals the brute force under each schedule; every schedule recovers the
  base model when s <= L; the factors are minimal by exhaustive check (parity of
  the variants' readings themselves unpinned: the pages print no value for them).
* ``bifocal_prefill_varlen``: each sequence's packed rows equal
  ``bifocal_bruteforce`` on its own rows and prefix, with the cache rows past the
  prefix set to NaN; a sequence with no new rows is skipped; with one sequence
  it equals ``bifocal_three_pass``.
* ``gather_pages`` / ``bifocal_decode_paged``: a contiguous cache scattered into
  shuffled pages (by the test, with NaN in every unused page) gathers back exactly,
  and the paged decode equals ``bifocal_decode_varlen`` / ``plain_decode_varlen``
  on the contiguous cache.
* ``sliding_window_attention``: torch's fp64 ``scaled_dot_product_attention`` with an
  explicit band mask; equals pass A of ``bifocal_three_pass``; equals
  ``plain_causal_attention`` when the window covers every key; W = 1 returns v_p.
* ``bifocal_decode_varlen`` / ``plain_decode_varlen``: each sequence equals
  ``bifocal_bruteforce`` (per-pair position selection, g from that sequence's own
  length) on its own prefix, with the cache rows past the prefix set to NaN; with
  every length <= L the two functions agree (exact recovery of the base model).

Where the pages are silent the reading taken is the plainest one the rest
supports; each is named where it is used.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "group_factor",
    "rope_frequencies",
    "rotate_half_pairs",
    "rotation_matrix",
    "aliased_position",
    "correction_offset",
    "query_positions",
    "plain_causal_attention",
    "bifocal_three_pass",
    "bifocal_bruteforce",
    "bifocal_decode",
    "bifocal_decode_varlen",
    "plain_decode_varlen",
    "bifocal_prefill_varlen",
    "gather_pages",
    "bifocal_decode_paged",
    "sliding_window_attention",
    "SCHEDULES",
    "seam_group_factor",
    "fractional_factor",
    "long_range_schedule",
    "merge_passes",
]


# ---------------------------------------------------------------------------
# Position rule
# ---------------------------------------------------------------------------

def group_factor(seq_len: int, pretrained_window: int) -> int:
    """Grouping factor g(s) by direct search.

    ResearchPod summary, 2nd paragraph: far keys are grouped by the least
    integer factor for which their rotation angles stay within what
    pretraining covered.  seventnews.com, "How bifocal attention sidesteps the
    fixed-scaling trap": the factor follows the length s of the sequence at
    hand.

    Reading: a key or query at position ``p < s`` is aliased to ``p // g``;
    pretraining saw positions (and distances) ``0 .. L-1``, so ``g`` is the
    smallest integer >= 1 with ``(s - 1) // g <= L - 1``.  This walks g upward
    and stops at the first one that satisfies the bound (deliberately not the
    closed form, which the tests compare against).
    """
    seq_len = int(seq_len)
    pretrained_window = int(pretrained_window)
    if seq_len < 1 or pretrained_window < 1:
        raise ValueError("seq_len and pretrained_window must be >= 1")
    g = 1
    while (seq_len - 1) // g > pretrained_window - 1:
        g += 1
    return g


def aliased_position(p, g: int):
    """a(p) = floor(p / g): a distant position mapped onto the pretrained grid
    (ResearchPod transcript, the exchange on position aliasing)."""
    return np.asarray(p, dtype=np.int64) // int(g)


def correction_offset(p, g: int):
    """c(p) = a(p) - p <= 0: the extra rotation that moves a vector cached at its
    original position p to its aliased position (ResearchPod transcript, the
    exchange on the cache: original positions are stored, the remapping is
    applied at lookup)."""
    p = np.asarray(p, dtype=np.int64)
    return p // int(g) - p


SCHEDULES = ("grouped", "seam", "fractional")


def seam_group_factor(seq_len: int, pretrained_window: int, local_window: int) -> int:
    """g for the seam-shifted grouping, by direct search: the smallest integer
    g >= 1 with ``(s-1) // g + W - W // g <= L - 1``, i.e. every remote query/key
    distance, shifted so that it continues the local window's distances at the
    seam, stays inside the pretrained positions.  Raises if no g does (W >= L
    with s > L)."""
    s, big_l, w = int(seq_len), int(pretrained_window), int(local_window)
    if s < 1 or big_l < 1 or w < 1:
        raise ValueError("sizes must be >= 1")
    for g in range(1, max(s, w) + 2):
        if (s - 1) // g + w - w // g <= big_l - 1:
            return g
    raise ValueError("no seam-shifted grouping keeps the distances inside the window (needs W < L)")


def fractional_factor(seq_len: int, pretrained_window: int) -> float:
    """l for the fractional scaling: the smallest real l >= 1 with
    ``(s - 1) / l <= L - 1``, the real-valued counterpart of the smallest integer
    grouping (seventnews.com, 1st section: a rescaling factor l(s) that follows
    the current length).  Needs L >= 2."""
    s, big_l = int(seq_len), int(pretrained_window)
    if s < 1 or big_l < 2:
        raise ValueError("need seq_len >= 1 and pretrained_window >= 2")
    return max(1.0, (s - 1) / (big_l - 1))


def long_range_schedule(seq_len: int, pretrained_window: int, local_window: int, schedule: str = "grouped"):
    """The positions a remote query and key are moved to, for one schedule.

    Returns ``(factor, a_q, a_k)``: the factor (integer g, or real l) and two
    functions mapping original positions to the positions used on the
    long-range branch.  The local branch always keeps the original positions.

    * ``grouped`` (the reading used everywhere else): a(p) = p // g on both sides
      (ResearchPod summary, 2nd paragraph: the least integer factor).
    * ``seam``: keys at j // g, queries at p // g + W - W // g.  The shift makes a
      remote distance continue the local window's distances at the seam; g grows
      to keep the shifted distances inside L.
    * ``fractional``: a(p) = p / l on both sides, the scaling read as a real
      factor (seventnews.com, 1st section; transform-ai's frequencies scaled
      dynamically).
    """
    if schedule == "grouped":
        g = group_factor(seq_len, pretrained_window)
        return g, (lambda p: np.asarray(p, dtype=np.int64) // g), (lambda j: np.asarray(j, dtype=np.int64) // g)
    if schedule == "seam":
        g = seam_group_factor(seq_len, pretrained_window, local_window)
        shift = int(local_window) - int(local_window) // g
        return (g, (lambda p: np.asarray(p, dtype=np.int64) // g + shift),
                (lambda j: np.asarray(j, dtype=np.int64) // g))
    if schedule == "fractional":
        lf = fractional_factor(seq_len, pretrained_window)
        return lf, (lambda p: np.asarray(p, dtype=np.float64) / lf), (lambda j: np.asarray(j, dtype=np.float64) / lf)
    raise ValueError(f"unknown schedule {schedule!r}")


def query_positions(n_q: int, n_kv: int, positions=None) -> np.ndarray:
    """Positions of the queries: the newest n_q tokens of an n_kv-key context, or
    the given ``positions`` (one per query row, each in [0, n_kv)): the queries of
    a chunk need not be contiguous nor the newest tokens."""
    if n_q > n_kv:
        raise ValueError("n_q must be <= n_kv")
    if positions is None:
        return np.arange(n_kv - n_q, n_kv, dtype=np.int64)
    pos = np.asarray(positions, dtype=np.int64)
    if pos.shape != (n_q,) or (n_q and (pos.min() < 0 or pos.max() >= n_kv)):
        raise ValueError("positions must hold one position in [0, n_kv) per query row")
    return pos


# ---------------------------------------------------------------------------
# RoPE (textbook definition; the pages name RoPE but print no formula)
# ---------------------------------------------------------------------------

def rope_frequencies(head_dim: int, rope_base: float) -> np.ndarray:
    """theta_d = base ** (-2 d / D), d = 0 .. D/2-1, in fp64."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    d = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(rope_base), -2.0 * d / head_dim)


def rotate_half_pairs(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate each pair (x_d, x_{d+D/2}) by angle phi_d (rotate-half convention):

        y_d       = x_d cos phi_d - x_{d+D/2} sin phi_d
        y_{d+D/2} = x_{d+D/2} cos phi_d + x_d sin phi_d

    ``angles`` has shape broadcastable to ``x[..., :D/2]``.
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    x1 = x[..., :h]
    x2 = x[..., h:]
    c = np.cos(angles)
    s = np.sin(angles)
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rotation_matrix(angles: np.ndarray) -> np.ndarray:
    """Explicit D x D block rotation R(phi) acting on rotate-half pairs, so that
    ``R @ x == rotate_half_pairs(x, phi)``.  Built entry by entry."""
    angles = np.asarray(angles, dtype=np.float64)
    h = angles.shape[0]
    r = np.zeros((2 * h, 2 * h), dtype=np.float64)
    for d in range(h):
        c = math.cos(angles[d])
        s = math.sin(angles[d])
        r[d, d] = c
        r[d, d + h] = -s
        r[d + h, d] = s
        r[d + h, d + h] = c
    return r


# ---------------------------------------------------------------------------
# Softmax pieces
# ---------------------------------------------------------------------------

def _partial_softmax(scores: np.ndarray, mask: np.ndarray, v: np.ndarray):
    """One FlashAttention-style pass restricted to ``mask``: returns the
    normalised partial output and its natural-log log-sum-exp.  An empty key
    set gives O = 0 and lse = -inf."""
    any_key = mask.any(axis=1)
    masked = np.where(mask, scores, -np.inf)
    m = masked.max(axis=1, initial=-np.inf)
    m_safe = np.where(any_key, m, 0.0)
    e = np.where(mask, np.exp(masked - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    l_safe = np.where(any_key, l, 1.0)
    out = (e @ v) / l_safe[:, None]
    out[~any_key] = 0.0
    lse = np.where(any_key, m_safe + np.log(l_safe), -np.inf)
    return out, lse


def merge_passes(o_a, lse_a, o_b, lse_b, o_c, lse_c):
    """Inclusion-exclusion merge of three passes (Abstract; ResearchPod summary,
    2nd paragraph; seventnews.com "How bifocal attention sidesteps the
    fixed-scaling trap": combined without double-counting).

    Pass B covers every causal key with grouped scores; pass C covers the local
    keys with the same grouped scores, so subtracting C removes the local keys'
    grouped contribution that B counted, and pass A puts them back with base
    scores:

        M = max(lse_A, lse_B, lse_C);  w_X = exp(lse_X - M)
        Z = w_A + w_B - w_C
        O = (w_A O_A + w_B O_B - w_C O_C) / Z;   lse = M + ln Z

    Outputs are ``[B, R, H, D]`` and log-sum-exps ``[B, H, R]``.
    """
    lses = np.stack([lse_a, lse_b, lse_c])
    m = np.max(lses, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)

    def w(lse):
        # weight per (B, H, R) -> laid out as (B, R, H, 1) to scale the outputs
        return np.swapaxes(np.where(np.isfinite(lse), np.exp(lse - m_safe), 0.0), 1, 2)

    w_a, w_b, w_c = w(lse_a), w(lse_b), w(lse_c)
    z = w_a + w_b - w_c
    out = (w_a[..., None] * o_a + w_b[..., None] * o_b - w_c[..., None] * o_c) / z[..., None]
    lse = m_safe + np.log(np.swapaxes(z, 1, 2))
    return out, lse


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, n, H, D]")
    b, n_q, hq, d = q.shape
    bk, n_kv, hkv, dk = k.shape
    if v.shape != k.shape or bk != b or dk != d:
        raise ValueError("shape mismatch")
    if hq % hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    if n_q > n_kv:
        raise ValueError("n_q must be <= n_kv")
    return b, n_q, n_kv, hq, hkv, d


# ---------------------------------------------------------------------------
# Plain causal attention (the base model; exact-recovery target)
# ---------------------------------------------------------------------------

def plain_causal_attention(q, k, v, softmax_scale=None, rows=None, row_block=256, positions=None):
    """Causal softmax attention on the cached (original-position) vectors.

    Returns ``(out [B, R, Hq, D], lse [B, Hq, R])`` for the selected query rows
    (all rows by default).  GQA: query head h reads KV head h // (Hq / Hkv).
    ``positions``: the query rows' positions (``query_positions``).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, n_q, n_kv, hq, hkv, d = _check_shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if not softmax_scale or softmax_scale <= 0 else float(softmax_scale)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = query_positions(n_q, n_kv, positions)
    grp = hq // hkv
    out = np.zeros((b, len(rows), hq, d))
    lse = np.zeros((b, hq, len(rows)))
    for bi in range(b):
        for h in range(hq):
            kh = h // grp
            for r0 in range(0, len(rows), row_block):
                sel = rows[r0:r0 + row_block]
                p = pos[sel]
                nk = int(p.max()) + 1
                s = scale * (q[bi, sel, h] @ k[bi, :nk, kh].T)
                j = np.arange(nk)
                mask = j[None, :] <= p[:, None]
                o, l_ = _partial_softmax(s, mask, v[bi, :nk, kh])
                out[bi, r0:r0 + len(sel), h] = o
                lse[bi, h, r0:r0 + len(sel)] = l_
    return out, lse


# ---------------------------------------------------------------------------
# O1: three-pass inclusion-exclusion form
# ---------------------------------------------------------------------------

def bifocal_three_pass(q, k, v, pretrained_window, local_window, rope_base,
                       softmax_scale=None, rows=None, row_block=128, schedule="grouped", positions=None):
    """Bifocal attention as three FlashAttention-style passes and their merge.

    ResearchPod summary, 2nd paragraph (three passes, the least integer factor);
    ResearchPod transcript, prefill exchange (near keys at base positions, all keys
    folded, near keys folded); ResearchPod transcript, cache exchange (keys kept at
    original positions, correction applied when read).

    Inputs are the cached vectors, already rotated at their original positions
    (``q`` at ``p_i``, ``k`` at ``j``).  Per query row i (position p_i):

    * Loc_i = {j : 0 <= p_i - j <= W - 1}  (W keys including the query itself),
      All_i = {j : j <= p_i}.
    * Pass A (near keys, base):    keys Loc_i, scores tau * q_i . k_j.
    * Pass B (all keys, folded):   keys All_i, scores tau * q^g_i . k^g_j with
      q^g_i = rot(q_i, c(p_i) theta), k^g_j = rot(k_j, c(j) theta).
    * Pass C (near keys, folded):  keys Loc_i, the grouped scores of pass B.
    * Merge: ``merge_passes``.

    Readings: absolute-position aliasing a(p) = p // g on both sides; no seam
    shift; g from s = n_kv; local iff p_i - j <= W - 1; tau = 1/sqrt(D) unless
    given; GQA head h -> KV head h // (Hq/Hkv).  ``schedule`` selects another
    long-range schedule (``long_range_schedule``): the corrections become
    rot(q, (a_q(p) - p) theta) and rot(k, (a_k(j) - j) theta).  ``positions``
    gives the query rows' positions (``query_positions``); g still comes from
    s = n_kv.

    Returns a dict with ``out [B, R, Hq, D]``, ``lse [B, Hq, R]`` (natural log),
    ``passes`` = {"A": (O, lse), "B": ..., "C": ...} with the same shapes, and
    ``g`` (the schedule's factor).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, n_q, n_kv, hq, hkv, d = _check_shapes(q, k, v)
    big_l = int(pretrained_window)
    w_loc = int(local_window)
    if w_loc < 1 or big_l < 1 or w_loc > big_l:
        raise ValueError("need 1 <= local_window <= pretrained_window")
    scale = 1.0 / math.sqrt(d) if not softmax_scale or softmax_scale <= 0 else float(softmax_scale)
    g, a_q, a_k = long_range_schedule(n_kv, big_l, w_loc, schedule)
    theta = rope_frequencies(d, rope_base)
    pos = query_positions(n_q, n_kv, positions)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    grp = hq // hkv

    # Correction rotations applied to the cached vectors (on the fly in the method).
    kpos = np.arange(n_kv, dtype=np.int64)
    k_corr = (a_k(kpos) - kpos).astype(np.float64)
    k_g = rotate_half_pairs(k, (k_corr[:, None] * theta)[None, :, None, :])
    q_sel_pos = pos[rows]
    q_sel = q[:, rows]
    q_corr = (a_q(q_sel_pos) - q_sel_pos).astype(np.float64)
    q_g = rotate_half_pairs(q_sel, (q_corr[:, None] * theta)[None, :, None, :])

    nr = len(rows)
    res = {x: (np.zeros((b, nr, hq, d)), np.zeros((b, hq, nr))) for x in "ABC"}
    for bi in range(b):
        for h in range(hq):
            kh = h // grp
            for r0 in range(0, nr, row_block):
                sl = slice(r0, r0 + row_block)
                p = q_sel_pos[sl]
                nk = int(p.max()) + 1
                j = np.arange(nk)
                dist = p[:, None] - j[None, :]
                causal = dist >= 0
                local = causal & (dist <= w_loc - 1)
                s_base = scale * (q_sel[bi, sl, h] @ k[bi, :nk, kh].T)
                s_grp = scale * (q_g[bi, sl, h] @ k_g[bi, :nk, kh].T)
                vv = v[bi, :nk, kh]
                for name, s_, m_ in (("A", s_base, local), ("B", s_grp, causal), ("C", s_grp, local)):
                    o, l_ = _partial_softmax(s_, m_, vv)
                    res[name][0][bi, sl, h] = o
                    res[name][1][bi, h, sl] = l_

    out, lse = merge_passes(res["A"][0], res["A"][1], res["B"][0], res["B"][1], res["C"][0], res["C"][1])
    return {"out": out, "lse": lse, "passes": res, "g": g}


def sliding_window_attention(q, k, v, local_window, softmax_scale=None, rows=None, row_block=256):
    """Plain sliding-window attention: query row i (position p_i) attends to the
    keys j with 0 <= p_i - j <= W - 1, scores tau * q_i . k_j on the cached
    vectors (base RoPE), one masked softmax per row.

    seventnews.com, "Generalization to hybrid attention architectures": hybrid
    models keep sliding-window layers next to the global ones.  A window W <= L
    never leaves the pretrained positions, so those layers run the base model's
    attention restricted to the window -- the local view (pass A) of the merge.
    Returns ``(out [B, R, Hq, D], lse [B, Hq, R])`` for the selected rows.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, n_q, n_kv, hq, hkv, d = _check_shapes(q, k, v)
    w_loc = int(local_window)
    if w_loc < 1:
        raise ValueError("need local_window >= 1")
    scale = 1.0 / math.sqrt(d) if not softmax_scale or softmax_scale <= 0 else float(softmax_scale)
    pos = query_positions(n_q, n_kv)
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    grp = hq // hkv
    out = np.zeros((b, len(rows), hq, d))
    lse = np.zeros((b, hq, len(rows)))
    for bi in range(b):
        for h in range(hq):
            kh = h // grp
            for r0 in range(0, len(rows), row_block):
                sl = slice(r0, r0 + row_block)
                p = pos[rows[sl]]
                lo = max(0, int(p.min()) - w_loc + 1)
                j = np.arange(lo, int(p.max()) + 1)
                dist = p[:, None] - j[None, :]
                band = (dist >= 0) & (dist <= w_loc - 1)
                s_ = scale * (q[bi, rows[sl], h] @ k[bi, lo:lo + len(j), kh].T)
                o, l_ = _partial_softmax(s_, band, v[bi, lo:lo + len(j), kh])
                out[bi, sl, h] = o
                lse[bi, h, sl] = l_
    return out, lse


# ---------------------------------------------------------------------------
# O2: brute-force per-pair position selection (tiny inputs only)
# ---------------------------------------------------------------------------

def _default_selection(g: int, local_window: int):
    def select(p: int, j: int):
        if p - j <= local_window - 1:
            return p, j              # local key: original positions, base RoPE
        return p // g, j // g        # remote key: both positions aliased
    return select


def bifocal_bruteforce(q_raw, k_raw, v, pretrained_window, local_window, rope_base,
                       softmax_scale=None, select=None, schedule="grouped", positions=None):
    """Bifocal attention written as one masked softmax with a per-pair choice of
    positions, on *raw* (un-rotated) q and k.  Pure Python loops over pairs and
    explicit D x D rotation matrices; for tiny inputs only.

    For each causal pair (i, j), j <= p_i: the local rule keeps the original
    positions (p_i, j) when p_i - j <= W-1 (ResearchPod transcript: nearby text
    keeps its original rotations); otherwise both positions are aliased to
    (p_i // g, j // g) (ResearchPod transcript: a far position is snapped to a
    coarser grid of positions seen in training).  Score
    ``tau * (R(P_q theta) q_i) . (R(P_k theta) k_j)``, explicit softmax over the
    row, output ``sum_j P_ij v_j``.

    ``select(p, j) -> (P_q, P_k)`` replaces the rule (tests use it to plant
    mistakes); by default the rule above with g = g(n_kv), or the remote
    positions (a_q(p), a_k(j)) of another ``schedule``.
    Returns ``(out [B, n_q, Hq, D], lse [B, Hq, n_q])``.
    """
    q_raw, k_raw, v = _as_f64(q_raw), _as_f64(k_raw), _as_f64(v)
    b, n_q, n_kv, hq, hkv, d = _check_shapes(q_raw, k_raw, v)
    scale = 1.0 / math.sqrt(d) if not softmax_scale or softmax_scale <= 0 else float(softmax_scale)
    if select is None and schedule == "grouped":
        select = _default_selection(group_factor(n_kv, pretrained_window), int(local_window))
    elif select is None:
        _, a_q, a_k = long_range_schedule(n_kv, pretrained_window, local_window, schedule)
        w_loc = int(local_window)

        def select(p: int, j: int):
            if p - j <= w_loc - 1:
                return p, j
            return float(a_q(p)), float(a_k(j))
    theta = rope_frequencies(d, rope_base)
    pos = query_positions(n_q, n_kv, positions)
    grp = hq // hkv
    mats = {}

    def rmat(position):
        if position not in mats:
            mats[position] = rotation_matrix(float(position) * theta)
        return mats[position]

    out = np.zeros((b, n_q, hq, d))
    lse = np.zeros((b, hq, n_q))
    for bi in range(b):
        for h in range(hq):
            kh = h // grp
            for i in range(n_q):
                p = int(pos[i])
                row = np.full(n_kv, -np.inf)
                for j in range(n_kv):
                    if j > p:
                        continue
                    pq, pk = select(p, j)
                    qr = rmat(pq) @ q_raw[bi, i, h]
                    kr = rmat(pk) @ k_raw[bi, j, kh]
                    row[j] = scale * float(qr @ kr)
                m = row.max()
                e = np.exp(row - m)
                z = e.sum()
                probs = e / z
                out[bi, i, h] = probs @ v[bi, :, kh]
                lse[bi, h, i] = m + math.log(z)
    return out, lse


# ---------------------------------------------------------------------------
# Decode: one new query against the original-position cache
# ---------------------------------------------------------------------------

def bifocal_decode(q, k_cache, v_cache, pretrained_window, local_window, rope_base,
                   softmax_scale=None, schedule="grouped"):
    """One generated token attending to a cache of n_kv keys that already holds
    its own key/value (ResearchPod transcript, cache exchange: original
    positions are stored; the correction happens at lookup).

    Reading: s = n_kv and the query sits at position n_kv - 1, so this is the
    last row of the three-pass prefill at the same s.  ``q`` is ``[B, 1, Hq, D]``.
    Returns ``(out [B, 1, Hq, D], lse [B, Hq, 1])``.
    """
    q = _as_f64(q)
    if q.shape[1] != 1:
        raise ValueError("decode takes one query row")
    r = bifocal_three_pass(q, k_cache, v_cache, pretrained_window, local_window, rope_base,
                           softmax_scale=softmax_scale, schedule=schedule)
    return r["out"], r["lse"]


def bifocal_decode_varlen(q, k_cache, v_cache, seq_lens, pretrained_window, local_window, rope_base,
                          softmax_scale=None):
    """A batch of sequences of different lengths, one new token each.  Sequence
    b holds the first ``seq_lens[b]`` rows of its cache at their original
    positions and its query sits at ``seq_lens[b] - 1``; the long-range factor
    is taken from that sequence's own length (seventnews.com, "How bifocal
    attention sidesteps the fixed-scaling trap": the factor follows the current
    length).  Each sequence is exactly the decode above on its own prefix.
    ``q`` is ``[B, 1, Hq, D]``, caches ``[B, N, Hkv, D]`` with N >= max(seq_lens).
    Returns ``(out [B, 1, Hq, D], lse [B, Hq, 1])``.
    """
    q = _as_f64(q)
    outs, lses = [], []
    for bi, s in enumerate(int(x) for x in seq_lens):
        o, l = bifocal_decode(q[bi:bi + 1], k_cache[bi:bi + 1, :s], v_cache[bi:bi + 1, :s], pretrained_window,
                              local_window, rope_base, softmax_scale=softmax_scale)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs, axis=0), np.concatenate(lses, axis=0)


def bifocal_prefill_varlen(q, cu_seqlens_q, k_cache, v_cache, seq_lens, pretrained_window, local_window,
                           rope_base, softmax_scale=None, schedule="grouped", bifocal=True):
    """A batch of sequences of different lengths, each with its own chunk of new
    queries against its own cache (the cache keeps original positions and the
    factor follows each sequence's current length: ResearchPod transcript, cache
    exchange; seventnews.com, "How bifocal attention sidesteps the fixed-scaling
    trap").  Sequence b owns the packed query rows ``cu_seqlens_q[b] ..
    cu_seqlens_q[b+1]-1`` of ``q [total_q, Hq, D]``, at positions ``s_b - n_b + i``
    with ``s_b = seq_lens[b]`` keys in rows 0 .. s_b-1 of ``k_cache, v_cache [B, N,
    Hkv, D]``.  Each sequence is exactly ``bifocal_three_pass`` (or plain causal
    attention with ``bifocal=False``) on its own rows and prefix.
    Returns ``(out [total_q, Hq, D], lse [Hq, total_q])``.
    """
    q = _as_f64(q)
    cu = [int(x) for x in cu_seqlens_q]
    hq, d = q.shape[1], q.shape[2]
    out = np.zeros((q.shape[0], hq, d))
    lse = np.zeros((hq, q.shape[0]))
    for bi, s in enumerate(int(x) for x in seq_lens):
        r0, r1 = cu[bi], cu[bi + 1]
        if r1 == r0:
            continue
        kb, vb = k_cache[bi:bi + 1, :s], v_cache[bi:bi + 1, :s]
        if bifocal:
            r = bifocal_three_pass(q[None, r0:r1], kb, vb, pretrained_window, local_window, rope_base,
                                   softmax_scale=softmax_scale, schedule=schedule)
            o, l = r["out"], r["lse"]
        else:
            o, l = plain_causal_attention(q[None, r0:r1], kb, vb, softmax_scale=softmax_scale)
        out[r0:r1] = o[0]
        lse[:, r0:r1] = l[0]
    return out, lse


def gather_pages(pages, block_table, seq_lens):
    """A paged cache as contiguous per-sequence caches: ``pages [n_pages, page_size,
    Hkv, D]``, ``block_table [B, pages_per_seq]``; position j of sequence b is row
    j % page_size of page block_table[b, j // page_size].  Returns ``[B,
    pages_per_seq * page_size, Hkv, D]`` with NaN past every sequence's length."""
    pages = np.asarray(pages)
    bt = np.asarray(block_table, dtype=np.int64)
    page_size = pages.shape[1]
    out = np.full((bt.shape[0], bt.shape[1] * page_size) + pages.shape[2:], np.nan)
    for bi, s in enumerate(int(x) for x in seq_lens):
        for j in range(s):
            out[bi, j] = pages[bt[bi, j // page_size], j % page_size]
    return out


def bifocal_decode_paged(q, k_pages, v_pages, block_table, seq_lens, pretrained_window, local_window, rope_base,
                         softmax_scale=None, schedule="grouped", bifocal=True):
    """Decode over a paged cache: the cache's pages are only a storage layout, so
    each sequence is exactly the decode on its gathered prefix (the keys keep their
    original positions: ResearchPod transcript, cache exchange).  ``q [B, 1, Hq,
    D]``; returns ``(out [B, 1, Hq, D], lse [B, Hq, 1])``."""
    k = gather_pages(_as_f64(k_pages), block_table, seq_lens)
    v = gather_pages(_as_f64(v_pages), block_table, seq_lens)
    q = _as_f64(q)
    outs, lses = [], []
    for bi, s in enumerate(int(x) for x in seq_lens):
        if bifocal:
            o, l = bifocal_decode(q[bi:bi + 1], k[bi:bi + 1, :s], v[bi:bi + 1, :s], pretrained_window, local_window,
                                  rope_base, softmax_scale=softmax_scale, schedule=schedule)
        else:
            o, l = plain_causal_attention(q[bi:bi + 1], k[bi:bi + 1, :s], v[bi:bi + 1, :s],
                                          softmax_scale=softmax_scale)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs, axis=0), np.concatenate(lses, axis=0)


def plain_decode_varlen(q, k_cache, v_cache, seq_lens, softmax_scale=None):
    """The base model's decode for a batch of sequences of different lengths:
    plain causal attention of the query at ``seq_lens[b] - 1`` over its own prefix."""
    q = _as_f64(q)
    outs, lses = [], []
    for bi, s in enumerate(int(x) for x in seq_lens):
        o, l = plain_causal_attention(q[bi:bi + 1], k_cache[bi:bi + 1, :s], v_cache[bi:bi + 1, :s],
                                      softmax_scale=softmax_scale)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs, axis=0), np.concatenate(lses, axis=0)
