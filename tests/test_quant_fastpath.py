"""The quantize kernels take each code from a reciprocal-multiply and fall
back to the IEEE division only inside a band around the ties.  This checks,
on the CPU and in binary32, that the band is wide enough: with the
reciprocal off by up to one ulp either way from the correctly rounded 1/scale
(v_rcp_f32 is documented to within 1 ulp of the exact reciprocal), the fast
path must give the code of the correctly rounded quotient,
round_half_even(fl32(fl32(x - mn) / scale)), for every value tried, at both
code widths.  It also shows that the band the kernels used before for every
width (2^-19) is too narrow at 4 bits, so the check has teeth.

The emulation restates the kernels' documented arithmetic; it calls neither
the HIP library nor the oracle.
"""
import numpy as np
import pytest

BAND = {2: 2.0 ** -19, 4: 2.0 ** -17}


def _rcp_variants(scale):
    r0 = (np.float32(1.0) / scale).astype(np.float32)
    up = np.nextafter(r0, np.float32(np.inf)).astype(np.float32)
    dn = np.nextafter(r0, np.float32(0.0)).astype(np.float32)
    return {"rn": r0, "up": up, "down": dn}


def _fast_codes(d, scale, rcp, band):
    """the kernels' code: rint(d * rcp), or rint(d / scale) within the band"""
    qa = (d * rcp).astype(np.float32)
    k = np.rint(qa)
    near = np.abs((qa - k).astype(np.float32)) > np.float32(0.5 - band)
    exact = np.rint((d / scale).astype(np.float32))
    return np.where(near, exact, k), near


def _groups(bits, rng, n_groups, n):
    """fp16 groups: Gaussian, outlier-scaled, narrow-exponent and random bit
    patterns, each with its group min / max and fp32 scale"""
    L = float((1 << bits) - 1)
    parts = []
    g = (rng.standard_normal((n_groups, n)).astype(np.float32)).astype(np.float16)
    parts.append(g)
    parts.append((rng.standard_normal((n_groups, n)).astype(np.float32) * 50).astype(np.float16))
    parts.append(rng.integers(0x3800, 0x4400, (n_groups, n)).astype(np.uint16).view(np.float16))
    bits_ = rng.integers(0, 0x7c00, (n_groups, n)).astype(np.uint16) | \
        (rng.integers(0, 2, (n_groups, n)).astype(np.uint16) << 15)
    parts.append(bits_.view(np.float16))
    x = np.concatenate(parts).astype(np.float32) + np.float32(0.0)   # -0 -> +0
    mn = x.min(axis=1, keepdims=True)
    mx = x.max(axis=1, keepdims=True)
    scale = ((mx - mn).astype(np.float32) / np.float32(L)).astype(np.float32)
    keep = scale[:, 0] > 0
    return x[keep], mn[keep], scale[keep]


def _near_tie_groups(bits, rng, n_groups):
    """groups whose members sit at and around the half-integer multiples of
    the scale: for a random fp16 range, every fp16 value within two ulps of
    (k + 1/2) * scale, k = 0 .. L - 1, shifted by a random fp16 minimum"""
    L = (1 << bits) - 1
    span = rng.integers(0x2000, 0x7800, n_groups).astype(np.uint16).view(np.float16).astype(np.float32)
    mn = rng.standard_normal(n_groups).astype(np.float16).astype(np.float32)
    mn = np.where(rng.random(n_groups) < 0.5, np.float32(0.0), mn)
    mx = (mn + span).astype(np.float16).astype(np.float32)
    ok = np.isfinite(mx) & (mx > mn)
    mn, mx = mn[ok], mx[ok]
    scale = ((mx - mn).astype(np.float32) / np.float32(L)).astype(np.float32)
    centre = (mn[:, None] + (np.arange(L)[None, :] + 0.5) * scale[:, None]).astype(np.float16)
    members = [centre]
    for toward in (np.float16(-np.inf), np.float16(np.inf)):
        m = centre
        for _ in range(2):
            m = np.nextafter(m, toward)
            members.append(m)
    x = np.concatenate(members, axis=1).astype(np.float32)
    x = np.clip(x, mn[:, None], mx[:, None]).astype(np.float32)
    assert np.isfinite(x).all()
    return x, mn[:, None], scale[:, None]


@pytest.mark.parametrize("bits", [2, 4])
def test_fast_path_exact_with_rcp_off_by_one_ulp(bits):
    rng = np.random.default_rng(0x51 + bits)
    checked = 0
    for x, mn, scale in (_groups(bits, rng, 40000, 32), _near_tie_groups(bits, rng, 200000)):
        d = (x - mn).astype(np.float32)
        want = np.rint((d / scale).astype(np.float32))
        for name, r in _rcp_variants(scale).items():
            got, _ = _fast_codes(d, scale, r, BAND[bits])
            bad = int(np.count_nonzero(got != want))
            assert bad == 0, (bits, name, bad)
        checked += d.size
    assert checked > 1_000_000


def test_old_band_fails_at_4_bits():
    """2^-19 is below the 4-bit bound 15 * 2^-22: some codes come out wrong
    once the reciprocal is one ulp off (at 2 bits the same band is exact, as
    the test above shows)."""
    rng = np.random.default_rng(0x77)
    x, mn, scale = _near_tie_groups(4, rng, 200000)
    d = (x - mn).astype(np.float32)
    want = np.rint((d / scale).astype(np.float32))
    wrong = 0
    for r in _rcp_variants(scale).values():
        got, _ = _fast_codes(d, scale, r, 2.0 ** -19)
        wrong += int(np.count_nonzero(got != want))
    assert wrong > 0


@pytest.mark.parametrize("bits", [2, 4])
def test_division_fallback_rate_on_gaussian_data(bits):
    """how often a code takes the IEEE division on the decode workloads'
    kind of data (N(0, 1) fp16, groups of 32): rare enough that a wave
    almost never waits for it"""
    rng = np.random.default_rng(0x99 + bits)
    x = rng.standard_normal((200000, 32)).astype(np.float32).astype(np.float16).astype(np.float32)
    mn = x.min(axis=1, keepdims=True)
    scale = ((x.max(axis=1, keepdims=True) - mn) / np.float32((1 << bits) - 1)).astype(np.float32)
    d = (x - mn).astype(np.float32)
    _, near = _fast_codes(d, scale, _rcp_variants(scale)["rn"], BAND[bits])
    rate = float(near.mean())
    print(f"bits {bits}: division fallback on {rate:.2e} of codes")
    assert rate < 1e-3
