"""Helpers for the GPU parity tests: device upload of the seeded bf16 inputs and
the parity bar against the fp64 oracle (bf16 inputs with fp32 accumulation):
outputs max-abs <= 1e-2 and mean-abs <= 1e-3.

The natural-log normaliser (lse) has a bar of its own (lse_tol).  Where every
score is taken on the vectors as given (plain attention, g = 1, sliding windows)
the kernels sum fp32 probabilities, so the lse carries fp32 rounding only and
the bar is 1e-3.  With g > 1 two further errors enter:
- grouped scores use q^g and k^g rounded to bf16 before the MFMA: each element
  carries a relative error of RMS ~1.6e-3 (round to nearest with 8 significant
  bits), which moves a score tau * q^g . k^g by ~1.6e-3 * sqrt(2 D) / sqrt(D) =
  2.3e-3 RMS for N(0, 1) inputs at D = 128;
- both bifocal forms (single kernel and two-launch) sum the bf16-rounded
  probabilities, the weights the P V product applies, so that each output is a
  convex combination of value rows: the normaliser's relative error is a
  weighted mean of roundings of at most 2^-8, RMS ~2.2e-3 at most.
The lse moves by the softmax-weighted mean of these errors, RMS up to
sqrt(2.3^2 + 2.2^2) e-3 * sqrt(sum_j p_j^2): 3.2e-3 only where one key holds all
the weight, far less once the weight is spread over the W + 1 or more keys of a
row with remote keys.  The bar is 4e-3; the largest lse error measured over
these tests is 1.6e-3.  The mean-abs bar stays 1e-3 for both.
"""

import numpy as np
import torch

MAX_ABS_TOL = 1e-2
MEAN_ABS_TOL = 1e-3
LSE_TOL_PLAIN = 1e-3    # scores on the vectors as given
LSE_TOL_GROUPED = 4e-3  # grouped scores on bf16-rounded corrected vectors
LSE_TOL = LSE_TOL_GROUPED
LSE_MEAN_TOL = MEAN_ABS_TOL


def lse_tol(g: int) -> float:
    """Max-abs bar of the lse for a call whose group factor is g (1: the base model)."""
    return LSE_TOL_PLAIN if g == 1 else LSE_TOL_GROUPED


def to_device(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit pattern -> contiguous torch.bfloat16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_parity(got: np.ndarray, ref: np.ndarray, what: str = "out", max_tol=MAX_ABS_TOL, mean_tol=MEAN_ABS_TOL):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    d = np.abs(got - ref)
    msg = f"{what}: max-abs {d.max():.3e} (tol {max_tol}), mean-abs {d.mean():.3e} (tol {mean_tol})"
    print(msg, flush=True)
    assert d.max() <= max_tol and d.mean() <= mean_tol, msg


def sample_rows(n_q: int, n_kv: int, big_l: int, w: int, g: int, count: int = 24, seed: int = 0) -> np.ndarray:
    """Rows that cover the interesting positions: first rows, the local/remote
    boundary p = W, positions next to multiples of g, the middle, the last rows,
    plus a few random ones."""
    off = n_kv - n_q
    rows = {0, 1, n_q - 1, n_q - 2, n_q // 2}
    for p in (w - 1, w, w + 1, big_l - 1, big_l, big_l + 1, 2 * big_l, n_kv - w, n_kv - 1):
        r = p - off
        if 0 <= r < n_q:
            rows.add(r)
    for k in range(1, 4):
        p = (n_kv // g - k) * g
        for dp in (-1, 0, 1):
            r = p + dp - off
            if 0 <= r < n_q:
                rows.add(r)
    rng = np.random.default_rng(seed)
    while len(rows) < count:
        rows.add(int(rng.integers(0, n_q)))
    return np.array(sorted(rows), dtype=np.int64)
