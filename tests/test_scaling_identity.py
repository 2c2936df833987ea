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


def test_double_reciprocal_product_exhaustive_at_workload_temperature(tmp_path):
    """Every non-NaN fp32 z (all 2^32 bit patterns) at T = 0.8, the
    temperature of the Qwen3-shaped workload's draw: the identity holds for
    the whole range, subnormal ties included (tests/scaling_exhaustive.c; run
    it by hand with other temperatures as arguments).  ~10 s of host time."""
    import os
    import shutil
    import subprocess

    import pytest

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "scaling_exhaustive.c")
    exe = str(tmp_path / "scaling_exhaustive")
    subprocess.run([cc, "-O2", "-o", exe, src], check=True)
    r = subprocess.run([exe, "0.8"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 mismatches" in r.stdout
