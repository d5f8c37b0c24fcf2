"""GPU parity of the decode over a paged cache against the fp64 oracle.

The keys and values of every sequence sit in pools of fixed-size pages, in an
order given by a table (shuffled here); positions, g and the schedule follow
each sequence's own length.  Unused pages and rows past a length hold NaN, so a
read outside a sequence's pages would poison its output.
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


def _paged_inputs(seed, lens, hq, hkv, page_size, spare_pages=3):
    b = len(lens)
    pages_per_seq = -(-max(lens) // page_size)
    n_pages = b * pages_per_seq + spare_pages
    rng = np.random.default_rng(seed)
    table = rng.permutation(n_pages)[:b * pages_per_seq].reshape(b, pages_per_seq).astype(np.int32)
    kp = np.full((n_pages, page_size, hkv, 128), BF16_NAN, dtype=np.uint16)
    vp = np.full_like(kp, BF16_NAN)
    kc = normal_bf16(seed, 1, (b, pages_per_seq * page_size, hkv, 128))
    vc = normal_bf16(seed, 2, (b, pages_per_seq * page_size, hkv, 128))
    for bi, s in enumerate(lens):
        for j0 in range(0, s, page_size):
            n = min(page_size, s - j0)
            kp[table[bi, j0 // page_size], :n] = kc[bi, j0:j0 + n]
            vp[table[bi, j0 // page_size], :n] = vc[bi, j0:j0 + n]
    qb = normal_bf16(seed, 0, (b, 1, hq, 128))
    return qb, kp, vp, table


def _run(qb, kp, vp, table, lens, big_l=None, w=None, base=None, schedule="grouped", plain=False):
    b, _, hq, _ = qb.shape
    page_size, hkv = kp.shape[1], kp.shape[2]
    q, kpd, vpd = to_device(qb), to_device(kp), to_device(vp)
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, 1), dtype=torch.float32, device="cuda:0")
    n_kv = table.shape[1] * page_size
    ws = torch.empty(jl.jl_bifocal_decode_workspace_size(b, n_kv, hq, hkv), dtype=torch.uint8, device="cuda:0")
    bt = torch.from_numpy(table).to("cuda:0")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda:0")
    print(f"paged decode lens={list(lens)} page={page_size} pages={kp.shape[0]} Hq={hq} Hkv={hkv} L={big_l} W={w} "
          f"schedule={schedule} plain={plain}", flush=True)
    if plain:
        jl.jl_plain_decode_paged(q, kpd, vpd, out, lse, bt, sl, ws)
    else:
        jl.jl_bifocal_decode_paged(q, kpd, vpd, out, lse, bt, sl, big_l, w, base, ws, schedule=schedule)
    torch.cuda.synchronize()
    return to_f64(out), lse.cpu().numpy().astype(np.float64)


def _oracle(qb, kp, vp, table, lens, big_l, w, base, schedule="grouped", plain=False):
    return oracle.bifocal_decode_paged(bf16_bits_to_f64(qb), bf16_bits_to_f64(kp), bf16_bits_to_f64(vp), table, lens,
                                       big_l, w, base, schedule=schedule, bifocal=not plain)


CASES = [
    # seed, lens, Hq, Hkv, page, L, W, base
    (1000, (1, 700, 1537, 3000), 8, 2, 32, 512, 128, 1e4),      # g = 1..6; the W boundary inside pages
    (1001, (3000, 129, 2048, 513), 8, 2, 64, 512, 100, 1e6),
    (1002, (4000, 4000), 16, 1, 256, 512, 500, 1e4),           # G = 16, W close to L
    (1003, (20000,), 32, 8, 128, 4096, 512, 1e6),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_paged_decode_parity(case):
    seed, lens, hq, hkv, ps, big_l, w, base = case
    qb, kp, vp, table = _paged_inputs(seed, list(lens), hq, hkv, ps)
    out, lse = _run(qb, kp, vp, table, lens, big_l, w, base)
    ro, rl = _oracle(qb, kp, vp, table, lens, big_l, w, base)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


@pytest.mark.parametrize("schedule", ["seam", "fractional"])
def test_paged_decode_schedules(schedule):
    lens = (1, 700, 1537, 3000)
    qb, kp, vp, table = _paged_inputs(1010, list(lens), 8, 2, 64)
    out, lse = _run(qb, kp, vp, table, lens, 512, 128, 1e4, schedule=schedule)
    ro, rl = _oracle(qb, kp, vp, table, lens, 512, 128, 1e4, schedule=schedule)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


def test_plain_paged_decode_parity():
    lens = (5, 1000, 2049)
    qb, kp, vp, table = _paged_inputs(1020, list(lens), 8, 2, 32)
    out, lse = _run(qb, kp, vp, table, lens, plain=True)
    ro, rl = _oracle(qb, kp, vp, table, lens, None, None, None, plain=True)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL_PLAIN, mean_tol=LSE_MEAN_TOL)


def test_paged_decode_128k_qwen3_shape():
    # the 128K Qwen3-8B decode head shape (32 / 8 heads, L = 32768, W = 4096) in pages of 256 positions
    lens = (131072, 65536)
    qb, kp, vp, table = _paged_inputs(1030, list(lens), 32, 8, 256, spare_pages=0)
    out, lse = _run(qb, kp, vp, table, lens, 32768, 4096, 1e6)
    ro, rl = _oracle(qb, kp, vp, table, lens, 32768, 4096, 1e6)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)


def test_paged_decode_wave_without_keys():
    # 131072 - 600 keys: the last chunk (1024 keys per chunk, 512 per wave here) holds 424,
    # so its second wave has no keys and re-reads the chunk's last key, which sits in an
    # earlier page than the wave's own start
    lens = (131072 - 600, 70001)
    qb, kp, vp, table = _paged_inputs(1040, list(lens), 32, 8, 256, spare_pages=2)
    out, lse = _run(qb, kp, vp, table, lens, 32768, 4096, 1e6)
    ro, rl = _oracle(qb, kp, vp, table, lens, 32768, 4096, 1e6)
    assert_parity(out, ro)
    assert_parity(lse, rl, "lse", max_tol=LSE_TOL, mean_tol=LSE_MEAN_TOL)
