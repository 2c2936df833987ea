"""The sampler kernels compute s = z / T as fl32(fl64(z) * fl64(1 / T)) when
|z| >= 2^-125 T, relying on that being the IEEE fp32 quotient (the double
product is within 2^-52 of z / T; an fp32 quotient that is not exact lies
more than 2^-49 from every fp32 rounding boundary outside the subnormal
range).  Checked here on the host against numpy's fp32 division, over
normal, scaled and extreme logits and temperatures."""
import numpy as np


def test_double_reciprocal_product_equals_fp32_division():
    rng = np.random.default_rng(5)
    temps = np.concatenate([
        np.array([0.8, 0.7, 1.0, 3.0, 6.0, 10.0, 0.01, 1e-30, 1e30, 3.4e38, 1.1754944e-38,
                  np.nextafter(np.float32(2), np.float32(0)), np.nextafter(np.float32(1), np.float32(2))],
                 np.float32),
        rng.uniform(0.05, 5.0, 24).astype(np.float32),
        (rng.integers(1, 2**31 - 2**23, 12).astype(np.uint32)).view(np.float32),
    ]).astype(np.float32)
    temps = temps[np.isfinite(temps) & (temps > 0)]
    z = np.concatenate([
        rng.standard_normal(200_000) * 3,
        rng.standard_normal(50_000) * 1e4,
        rng.standard_normal(50_000) * 1e-30,
        rng.integers(-2**24, 2**24, 50_000).astype(np.float64),
    ]).astype(np.float32)
    z = np.concatenate([z, rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    z = z[np.isfinite(z)]
    checked = 0
    with np.errstate(over="ignore", under="ignore"):
        for T in temps:
            use = np.abs(z) >= T * np.float32(2.0 ** -125)
            zz = z[use]
            div = zz / T
            prod = (zz.astype(np.float64) * (1.0 / np.float64(T))).astype(np.float32)
            assert np.array_equal(div.view(np.uint32), prod.view(np.uint32)), float(T)
            checked += zz.size
    assert checked > 10_000_000
