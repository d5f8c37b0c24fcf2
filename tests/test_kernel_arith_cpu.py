"""Integer shortcuts the HIP kernels take, checked exhaustively on the CPU.

The single-kernel bifocal prefill indexes its small-angle rotation table with
u = kt - floor((r + kt) / g), r = j0 mod g, kt < 64, and forms that floor
without a division: n for g = 1, the high word of n * ceil(2^32 / g) for
2 <= g <= 65472, and n >= g above (where n < 2g).  The multiply-high form is
exact while n g < 2^32; these tests check every n the kernel can present for
every g up to 4096 and around the switch-over, plus the claimed bound on u.
The per-tile scalars (j0 mod g, floor(j0 / g)) are advanced by adding the
quotient and remainder of 64 / g once per tile; that recurrence is checked
against direct division too."""

import numpy as np

MAGIC_MAX_G = 65472
TILE = 64


def floor_div(n, g):
    n = np.asarray(n, dtype=np.uint64)
    if g == 1:
        return n
    if g <= MAGIC_MAX_G:
        m = np.uint64(((1 << 32) + g - 1) // g)
        return (n * m) >> np.uint64(32)
    return (n >= g).astype(np.uint64)


def check_g(g):
    # n = r + kt with r = j0 mod g in [0, g), kt in [0, 64)
    n = np.arange(0, g + TILE - 1, dtype=np.uint64)
    got = floor_div(n, g)
    assert np.array_equal(got, n // np.uint64(g)), g
    r = np.arange(g, dtype=np.int64)[:, None]
    kt = np.arange(TILE, dtype=np.int64)[None, :]
    u = kt - (r + kt) // g
    assert u.min() >= 0 and u.max() < TILE, g


def test_floor_div_small_g_exhaustive():
    for g in range(1, 4097):
        check_g(g)


def test_floor_div_around_the_switch_over():
    for g in list(range(MAGIC_MAX_G - 64, MAGIC_MAX_G + 65)) + [1 << 17, (1 << 30)]:
        if g > 1 << 20:
            # n < 2g: only the neighbourhood of g can give 1
            n = np.array([0, 1, g - 64, g - 1, g, g + 1, g + 62], dtype=np.uint64)
            assert np.array_equal(floor_div(n, g), n // np.uint64(g)), g
        else:
            check_g(g)


def test_magic_bound_holds_up_to_the_switch_over():
    # n <= g + 63, exactness needs n g < 2^32
    assert (MAGIC_MAX_G + 63) * MAGIC_MAX_G < 1 << 32


def test_per_tile_scalars_recurrence():
    for g in [1, 2, 3, 4, 5, 7, 31, 63, 64, 65, 100, 4096, 1 << 30]:
        r64, q64 = TILE % g, TILE // g
        r, q = 0, 0
        for t in range(1, 300):
            r += r64
            q += q64
            if r >= g:
                r -= g
                q += 1
            j0 = t * TILE
            assert (r, q) == (j0 % g, j0 // g), (g, t)
