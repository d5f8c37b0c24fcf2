"""Helpers for the GPU parity tests: device upload of the seeded bf16 inputs and
the parity bar (max-abs <= 1e-2 and mean-abs <= 1e-3 against the fp64 oracle,
bf16 inputs with fp32 accumulation).

The same bar applies to the natural-log normaliser (lse).  Its error is set by
the scores: the corrected vectors q^g and k^g are rounded to bf16 before the
MFMA (relative error up to 2^-8 per element, bf16's unit roundoff), which moves a grouped score
tau * q^g . k^g by ~2e-3 RMS for N(0,1) inputs at D = 128, and the lse of a short
row inherits that directly."""

import numpy as np
import torch

MAX_ABS_TOL = 1e-2
MEAN_ABS_TOL = 1e-3
LSE_TOL = MAX_ABS_TOL
LSE_MEAN_TOL = MEAN_ABS_TOL


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
