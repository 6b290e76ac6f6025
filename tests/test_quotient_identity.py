"""The FP8 quantiser divides by the block descale as (float)((double)y * (1.0 / (double)descale)).
This CPU check pins the claim that this equals the IEEE fp32 quotient y / descale bit for bit:
the fp64 product is within 2^-52 (relative) of y/descale, and a quotient of two fp32 numbers
is never that close to an fp32 rounding boundary. Random operands over all mantissa patterns
(including all-ones and near-power-of-two divisors) and the quotient range the quantiser uses
(|y / descale| <= 448)."""
import numpy as np


def test_fp64_reciprocal_product_rounds_like_fp32_division():
    rng = np.random.default_rng(2024)
    n = 1_000_000
    for mode in range(3):
        bits = rng.integers(0, 2 ** 23, n, dtype=np.uint32)
        if mode == 1:
            bits = (2 ** 23 - 1) - rng.integers(0, 64, n, dtype=np.uint32)
        elif mode == 2:
            bits = rng.integers(0, 64, n, dtype=np.uint32)
        exps = rng.integers(60, 190, n, dtype=np.uint32)
        ds = ((exps << 23) | bits).view(np.float32)
        yexp = (exps.astype(np.int64) + rng.integers(-40, 9, n)).clip(1, 254).astype(np.uint32)
        y = ((yexp << 23) | rng.integers(0, 2 ** 23, n, dtype=np.uint32)).view(np.float32)
        y = y * np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32)
        ref = y / ds
        got = (y.astype(np.float64) * (1.0 / ds.astype(np.float64))).astype(np.float32)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
