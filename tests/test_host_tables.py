"""The library's host precompute of the per-band constants (tria_band_tables, the values
tria_load_calib builds its device table from) against a 50-digit mpmath reference, on the CPU.

  C_f, S_f  the offset means of cos / sin(w_f d) over D (chenxutan.com/d/2624 section 3.3):
            within 4e-16 of the mean of the exact cosines and sines of w_f d, w_f taken as the
            exact binary value the library uses (fl32 of the fp64 power);
  nu_f      w_f / 2pi as a 64-bit fraction of a turn: within one unit of round(w_f / 2pi 2^64);
            the phase t nu mod 2^64 of a position t < 2^31 is within 2^-31 turns of frac(t w_f / 2pi).
"""
import mpmath
import numpy as np
import pytest

mp = mpmath.mp


@pytest.fixture(scope="module")
def T():
    import kv_cache_compression_tria_amd as T
    T.lib()
    return T


def reference(w, offsets):
    mp.dps = 50
    C, S, nu = [], [], []
    for wf in w:
        x = mpmath.mpf(float(wf))            # the exact binary value
        C.append(mpmath.fsum(mpmath.cos(x * d) for d in offsets) / len(offsets))
        S.append(mpmath.fsum(mpmath.sin(x * d) for d in offsets) / len(offsets))
        nu.append(int(mpmath.nint(x / (2 * mpmath.pi) * mpmath.mpf(2) ** 64)))
    return C, S, nu


@pytest.mark.parametrize("theta,offsets", [(1e6, None), (1e4, None), (1e6, [0, 3, 1000, 65535, 2 ** 24 - 1])])
def test_band_tables_against_mpmath(T, theta, offsets):
    w, C, S, nu = T.band_tables(theta, 128, offsets)
    D = [2 ** i for i in range(17)] if offsets is None else offsets
    # w_f: the fp64 power rounded once to fp32
    f = np.arange(64, dtype=np.float64)
    assert np.array_equal(w, np.power(theta, -2.0 * f / 128).astype(np.float32).astype(np.float64))
    Cr, Sr, nur = reference(w, D)
    for i in range(64):
        assert abs(C[i] - float(Cr[i])) <= 4e-16, (i, C[i], Cr[i])
        assert abs(S[i] - float(Sr[i])) <= 4e-16, (i, S[i], Sr[i])
        assert abs(int(nu[i]) - nur[i]) <= 1, (i, int(nu[i]), nur[i])


def test_turn_fraction_phases(T):
    w, _, _, nu = T.band_tables(1e6, 128)
    mp.dps = 60
    for i in (0, 1, 17, 40, 63):
        x = mpmath.mpf(float(w[i]))
        for t in (0, 1, 4000, 32767, 2 ** 24 - 1, 2 ** 31 - 1):
            lib_turns = mpmath.mpf((t * int(nu[i])) % 2 ** 64) / mpmath.mpf(2) ** 64
            exact = mpmath.frac(t * x / (2 * mpmath.pi))
            dist = abs(lib_turns - exact)
            dist = min(dist, 1 - dist)                # on the circle
            assert dist <= mpmath.mpf(2) ** -31, (i, t, float(dist))


def test_band_tables_errors(T):
    with pytest.raises(T.TriaError) as e:
        T.band_tables(1e6, 64)
    assert e.value.status == T.E_UNSUPPORTED
    for theta, off in ((1.0, None), (float("inf"), None), (1e6, [2 ** 24]), (1e6, [-1])):
        with pytest.raises(T.TriaError) as e:
            T.band_tables(theta, 128, off)
        assert e.value.status == T.E_INVALID
