"""Pins of the fp64 oracle against facts the pages and the mathematics fix (CPU only).

Each test states what it pins.  None of them re-types the oracle's own formula: the
trigonometric score is checked against RoPE'd dot products built here with numpy, against
closed forms worked by hand, and against invariants of the z-score and of top-B selection.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import synth

D_DEF = synth.OFFSETS
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def np_rope(x, p, w):
    """Half-split RoPE of vectors x [..., d] at integer positions p (fp64, written for the test)."""
    h = x.shape[-1] // 2
    a = np.asarray(p, dtype=np.float64)[..., None] * w
    c, s = np.cos(a), np.sin(a)
    return np.concatenate([x[..., :h] * c - x[..., h:] * s, x[..., :h] * s + x[..., h:] * c], axis=-1)


def rand_stream(rng, N, d, G, t, dtype="f32", concentrated=True):
    w = synth.omega_table(d)
    if concentrated:
        c = 8 * rng.standard_normal(d) / math.sqrt(d)
        pre = c + 0.5 * rng.standard_normal((N, d))
    else:
        pre = rng.standard_normal((N, d))
    pos = np.sort(rng.choice(t + 1, size=N, replace=False)).astype(np.int32)
    post = np_rope(pre, pos, w).astype(np.float32)
    keys = post if dtype == "f32" else synth.f32_to_bf16_bits(post)
    qc = (8 * rng.standard_normal((G, d)) / math.sqrt(d)).astype(np.float32)
    qn = rng.uniform(0.5, 2.0, (G, d // 2)).astype(np.float32)
    rb = rng.uniform(0.6, 0.99, (G, d // 2)).astype(np.float32)
    return keys, pos, qc, qn, rb


def keys_f64(keys):
    return (synth.bf16_bits_to_f32(keys) if keys.dtype == np.uint16 else keys).astype(np.float64)


# ---- P1: the trig series equals the offset-averaged RoPE'd centre-key dot product ---------------

@pytest.mark.parametrize("form", ["lit", "fac"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p1_trig_series_is_rope_dot_product(orc, form, dtype):
    """When the query equals its centre, the trigonometric series is exactly the mean over the
    future offsets of <RoPE(qbar, t+d), ktilde_j> (the derivation on the TriAttention pages:
    zhichai.net "三角函数的魔法", chenxutan.com/d/2624 section 3.1).  Pins the band layout,
    the sign of the distance, the phase recovery and the offset mean."""
    rng = np.random.default_rng(11)
    d, G, N, t = 128, 3, 40, 5000
    keys, pos, qc, qn, rb = rand_stream(rng, N, d, G, t, dtype)
    w = synth.omega_table(d)
    kt = keys_f64(keys)
    st, sn, raw = orc.score_stream(keys, pos, t, qc, qn, rb, form=form)
    expect = np.zeros((G, N))
    scale = np.zeros((G, N))
    for dd in D_DEF:
        qrot = np_rope(qc.astype(np.float64), t + dd, w)     # [G][d]
        expect += qrot @ kt.T
        scale += np.abs(qrot) @ np.abs(kt).T
    expect /= len(D_DEF)
    scale /= len(D_DEF)
    assert np.max(np.abs(st - expect) / scale) < 1e-12
    np.testing.assert_allclose(raw, st + sn, rtol=0, atol=1e-12 * np.max(np.abs(raw)))


def test_p1_large_positions(orc):
    """Same identity at positions near 2^17 and with the slowest and fastest bands dominant."""
    rng = np.random.default_rng(12)
    d, G, N, t = 128, 2, 16, 131000 - 65536
    keys, pos, qc, qn, rb = rand_stream(rng, N, d, G, t, "f32", concentrated=False)
    w = synth.omega_table(d)
    kt = keys_f64(keys)
    for form in ("lit", "fac"):
        st, _, _ = orc.score_stream(keys, pos, t, qc, qn, rb, form=form)
        expect = sum(np_rope(qc.astype(np.float64), t + dd, w) @ kt.T for dd in D_DEF) / len(D_DEF)
        scale = sum(np.abs(np_rope(qc.astype(np.float64), t + dd, w)) @ np.abs(kt).T for dd in D_DEF) / len(D_DEF)
        assert np.max(np.abs(st - expect) / scale) < 1e-11


# ---- P2: R = 1 removes the norm score ----------------------------------------------------------

def test_p2_r_one_zeroes_norm(orc):
    """The norm score carries the weight (1 - R) (10100.com "TriAttention方法"; watermelonwater.tech
    "TriAttention 方案设计"): R_f = 1 for every band leaves exactly the trigonometric score."""
    rng = np.random.default_rng(2)
    keys, pos, qc, qn, rb = rand_stream(rng, 64, 128, 4, 3000, "bf16")
    st, sn, raw = orc.score_stream(keys, pos, 3000, qc, qn, np.ones_like(rb))
    assert np.all(sn == 0.0)
    assert np.array_equal(raw, st)


def test_norm_score_closed_form(orc):
    """S_norm = sum_f (1-R_f) E|q_f| |k_f| with |k_f| the band magnitude of the stored key
    (RoPE preserves band norms).  Built here from the stored key directly, without phase recovery."""
    rng = np.random.default_rng(3)
    keys, pos, qc, qn, rb = rand_stream(rng, 50, 128, 2, 7000, "f32")
    _, sn, _ = orc.score_stream(keys, pos, 7000, qc, qn, rb)
    kt = keys_f64(keys)
    mag = np.hypot(kt[:, :64], kt[:, 64:])
    expect = ((1 - rb.astype(np.float64)) * qn.astype(np.float64)) @ mag.T
    np.testing.assert_allclose(sn, expect, rtol=1e-13)


# ---- P6: special cases that reduce to a textbook dot product -----------------------------------

def test_p6_zero_offset_at_key_position_is_plain_dot(orc):
    """D = {0} and p_j = t: the score is the plain pre-RoPE dot product <qbar, k_j>."""
    rng = np.random.default_rng(6)
    d, G, N, t = 128, 2, 10, 12345
    w = synth.omega_table(d)
    post = rng.standard_normal((N, d)).astype(np.float32)
    pos = np.full(N, t, dtype=np.int32)
    pre = np_rope(post.astype(np.float64), -t, w)          # exact inverse rotation of the stored key
    qc = rng.standard_normal((G, d)).astype(np.float32)
    qn = np.ones((G, d // 2), np.float32)
    rb = np.ones((G, d // 2), np.float32)
    for form in ("lit", "fac"):
        st, _, _ = orc.score_stream(post, pos, t, qc, qn, rb, offsets=(0,), form=form)
        expect = qc.astype(np.float64) @ pre.T
        np.testing.assert_allclose(st, expect, rtol=0, atol=1e-12 * np.abs(qc).sum() * np.abs(pre).max())


def test_p6_zero_offset_any_position_is_rotated_query_dot(orc):
    """D = {0}, arbitrary positions: the score is <RoPE(qbar, t), ktilde_j>."""
    rng = np.random.default_rng(7)
    d, G, N, t = 128, 3, 12, 9000
    w = synth.omega_table(d)
    post = rng.standard_normal((N, d)).astype(np.float32)
    pos = rng.integers(0, t + 1, N).astype(np.int32)
    qc = rng.standard_normal((G, d)).astype(np.float32)
    ones = np.ones((G, d // 2), np.float32)
    st, _, _ = orc.score_stream(post, pos, t, qc, ones, ones, offsets=(0,), form="lit")
    expect = np_rope(qc.astype(np.float64), t, w) @ post.astype(np.float64).T
    np.testing.assert_allclose(st, expect, rtol=0, atol=1e-11)


# ---- P7: one band, closed form ------------------------------------------------------------------

@pytest.mark.parametrize("f", [0, 1, 17, 63])
def test_p7_single_band_closed_form(orc, f):
    """Only band f non-zero: S = |q_f||k_f| mean_d cos(w_f (t+d-p) + phi), worked with cmath.
    Band 0 has w = 1 exactly, so w*d reaches 65536 rad."""
    d, t = 128, 4000
    w = synth.omega_table(d)
    assert w[0] == 1.0
    qc = np.zeros((1, d), np.float32)
    qc[0, f], qc[0, f + 64] = 0.75, -1.25
    post = np.zeros((3, d), np.float32)
    post[:, f] = [2.0, -0.5, 1.5]
    post[:, f + 64] = [1.0, 3.0, -0.25]
    pos = np.array([0, 1234, 3999], np.int32)
    ones = np.ones((1, 64), np.float32)
    for form in ("lit", "fac"):
        st, _, _ = orc.score_stream(post, pos, t, qc, ones, ones, form=form)
        for j in range(3):
            q = complex(0.75, -1.25)
            kt = complex(float(post[j, f]), float(post[j, f + 64]))
            k = kt * complex(math.cos(w[f] * pos[j]), -math.sin(w[f] * pos[j]))
            val = sum(abs(q) * abs(k) * math.cos(w[f] * (t + dd - int(pos[j])) + math.atan2(q.imag, q.real)
                                                 - math.atan2(k.imag, k.real)) for dd in D_DEF) / len(D_DEF)
            assert abs(st[0, j] - val) < 1e-12 * abs(q) * abs(k)


def test_golden_hand_cases(orc):
    """Hand-worked cases in tests/golden/hand_cases.json (d = 2 or 4; w_0 = 1 for any theta)."""
    with open(os.path.join(GOLDEN, "hand_cases.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        keys = np.array(c["keys"], np.float32)
        st, sn, raw = orc.score_stream(keys, np.array(c["pos"], np.int32), c["t"],
                                       np.array(c["qc"], np.float32), np.array(c["qn"], np.float32),
                                       np.array(c["rb"], np.float32), theta=c["theta"],
                                       offsets=tuple(c["offsets"]), form="lit")
        np.testing.assert_allclose(raw.ravel(), np.array(eval(c["expect_expr"], {"math": math})).ravel(),
                                   rtol=1e-13, atol=1e-13, err_msg=c["name"])


# ---- P10: factored form equals the literal form -------------------------------------------------

def test_p10_fac_equals_lit(orc):
    rng = np.random.default_rng(10)
    keys, pos, qc, qn, rb = rand_stream(rng, 200, 128, 4, 16383, "bf16")
    a = orc.score_stream(keys, pos, 16383, qc, qn, rb, form="lit")
    b = orc.score_stream(keys, pos, 16383, qc, qn, rb, form="fac")
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-12 * np.max(np.abs(x))


# ---- P11: keys cached before RoPE ---------------------------------------------------------------

@pytest.mark.parametrize("form", ["lit", "fac"])
def test_p11_pre_rope_keys_zero_offset_is_rope_dot(orc, form):
    """Pre-RoPE keys, D = {0}: the score is <RoPE(qbar, t), RoPE(k_j, p_j)>, both rotations done
    here with numpy (the trig series depends on the key only through its pre-RoPE bands)."""
    rng = np.random.default_rng(111)
    d, G, N, t = 128, 3, 16, 20000
    w = synth.omega_table(d)
    pre = rng.standard_normal((N, d)).astype(np.float32)
    pos = rng.integers(0, t + 1, N).astype(np.int32)
    qc = rng.standard_normal((G, d)).astype(np.float32)
    ones = np.ones((G, d // 2), np.float32)
    st, _, _ = orc.score_stream(pre, pos, t, qc, ones, ones, offsets=(0,), form=form, pre_rope=True)
    expect = np_rope(qc.astype(np.float64), t, w) @ np_rope(pre.astype(np.float64), pos, w).T
    # angles reach 2e4 rad (band 0 has w = 1): each fp64 cos/sin of them is good to ~4e-12, and
    # 64 bands of |q||k| ~ 1 add up to a few 1e-11
    np.testing.assert_allclose(st, expect, rtol=0, atol=1e-10)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p11_pre_rope_equals_post_rope_of_same_keys(orc, dtype):
    """The same pre-RoPE keys scored directly and after a RoPE done here (fp64, rounded to fp32):
    every score agrees to the rounding of the stored post-RoPE keys (relative 1e-6), and the
    norm scores agree too (|k_f| is RoPE-invariant)."""
    rng = np.random.default_rng(112)
    d, G, N, t = 128, 4, 60, 30000
    w = synth.omega_table(d)
    pre32 = (1.5 * rng.standard_normal(d) + rng.standard_normal((N, d))).astype(np.float32)
    keys = pre32 if dtype == "f32" else synth.f32_to_bf16_bits(pre32)
    pos = np.sort(rng.choice(t + 1, size=N, replace=False)).astype(np.int32)
    post = np_rope(keys_f64(keys), pos, w).astype(np.float32)
    qc = (8 * rng.standard_normal((G, d)) / math.sqrt(d)).astype(np.float32)
    qn = rng.uniform(0.5, 2.0, (G, d // 2)).astype(np.float32)
    rb = rng.uniform(0.6, 0.99, (G, d // 2)).astype(np.float32)
    a = orc.score_stream(keys, pos, t, qc, qn, rb, form="fac", pre_rope=True)
    b = orc.score_stream(post, pos, t, qc, qn, rb, form="fac")
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-6 * np.max(np.abs(x))


def test_p11_pre_rope_single_band_closed_form(orc):
    """Pre-RoPE keys, one band: S = |q_f||k_f| mean_d cos(w_f (t+d-p) + arg q - arg k) with k
    taken as stored (no phase recovery), worked with cmath."""
    d, t, f = 128, 4000, 9
    w = synth.omega_table(d)
    qc = np.zeros((1, d), np.float32)
    qc[0, f], qc[0, f + 64] = -0.5, 2.0
    pre = np.zeros((2, d), np.float32)
    pre[:, f] = [1.25, -3.0]
    pre[:, f + 64] = [0.5, 0.75]
    pos = np.array([17, 3998], np.int32)
    ones = np.ones((1, 64), np.float32)
    st, _, _ = orc.score_stream(pre, pos, t, qc, ones, ones, form="lit", pre_rope=True)
    q = complex(-0.5, 2.0)
    for j in range(2):
        k = complex(float(pre[j, f]), float(pre[j, f + 64]))
        val = sum(abs(q) * abs(k) * math.cos(w[f] * (t + dd - int(pos[j])) + math.atan2(q.imag, q.real)
                                             - math.atan2(k.imag, k.real)) for dd in D_DEF) / len(D_DEF)
        assert abs(st[0, j] - val) < 1e-12 * abs(q) * abs(k)


# ---- z-score and GQA max ------------------------------------------------------------------------

def test_zscore_moments_and_max(orc):
    """Per head, z has mean 0 and population std 1; F is the max over the group
    (10100.com "TriAttention方法"; watermelonwater.tech "TriAttention 方案设计" item 4)."""
    rng = np.random.default_rng(4)
    raw = rng.standard_normal((5, 301)) * rng.uniform(0.1, 30, (5, 1)) + rng.uniform(-50, 50, (5, 1))
    z, F, mu, sd = orc.zmax(raw)
    np.testing.assert_allclose(z.mean(axis=1), 0, atol=1e-13)
    np.testing.assert_allclose(z.std(axis=1), 1, atol=1e-13)
    np.testing.assert_array_equal(F, z.max(axis=0))
    np.testing.assert_allclose(mu, raw.mean(axis=1), rtol=1e-14)


def test_zscore_shift_and_scale_invariance(orc):
    rng = np.random.default_rng(5)
    raw = rng.standard_normal((3, 100))
    _, F1, _, _ = orc.zmax(raw)
    _, F2, _, _ = orc.zmax(raw * 7.5 + 3.25)
    np.testing.assert_allclose(F1, F2, atol=1e-13)


def test_zscore_constant_head(orc):
    """A head whose scores are all equal has std 0 and contributes z = 0."""
    raw = np.vstack([np.full(10, 3.0), np.linspace(-1, 1, 10)])
    z, F, mu, sd = orc.zmax(raw)
    assert sd[0] == 0.0 and np.all(z[0] == 0.0)
    np.testing.assert_array_equal(F, np.maximum(z[1], 0.0))


def test_zscore_rounding_level_spread_is_constant(orc):
    """Scores equal up to rounding (spread <= 2^-16 of their magnitude) count as constant."""
    base = 7.25
    raw = np.vstack([base * (1 + np.linspace(-1, 1, 9) * 2.0 ** -18), np.linspace(-1, 1, 9)])
    z, F, mu, sd = orc.zmax(raw)
    assert sd[0] == 0.0 and np.all(z[0] == 0.0)
    raw2 = np.vstack([base * (1 + np.linspace(-1, 1, 9) * 2.0 ** -12), np.linspace(-1, 1, 9)])
    z2, _, _, sd2 = orc.zmax(raw2)
    assert sd2[0] > 0.0
    np.testing.assert_allclose(z2[0], z2[1], atol=1e-9)


def test_zscore_nonfinite_raises(orc):
    raw = np.ones((1, 4))
    raw[0, 2] = np.nan
    with pytest.raises(ValueError):
        orc.zmax(raw)


# ---- P3 / P4 / P5 / P8: selection --------------------------------------------------------------

def brute_force_topB(F, B):
    """Among all B-subsets: maximal sum of F, then lexicographically least sorted index tuple."""
    best = None
    for comb in itertools.combinations(range(len(F)), B):
        s = sum(F[i] for i in comb)
        if best is None or s > best[0] + 1e-12 or (abs(s - best[0]) <= 1e-12 and comb < best[1]):
            best = (s, comb)
    return list(best[1])


@pytest.mark.parametrize("seed", range(6))
def test_p3_select_matches_brute_force(orc, seed):
    """Top-B (torch.topk then sort in chenxutan.com/d/2624 section 4.2) equals the brute-force
    optimum on tiny inputs, with ties resolved to the lower index."""
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 12))
    F = rng.integers(-3, 4, N).astype(np.float64) * 0.5   # many ties
    for B in range(1, N + 1):
        got = list(orc.select(F, B))
        assert got == brute_force_topB(F, B), (F, B)


def test_select_negative_zero_ties_with_zero(orc):
    F = np.array([0.0, -0.0, 0.0, -0.0, -1.0])
    assert list(orc.select(F, 2)) == [0, 1]
    assert list(orc.select(F, 3)) == [0, 1, 2]


def test_p8_budget_at_least_n_is_identity(orc):
    F = np.random.default_rng(8).standard_normal(37)
    assert list(orc.select(F, 37)) == list(range(37))
    assert list(orc.select(F, 100)) == list(range(37))
    rows = np.arange(37 * 4, dtype=np.int32).reshape(37, 4)
    np.testing.assert_array_equal(orc.compact_rows(rows, np.arange(37)), rows)


def test_p4_single_head_selects_top_raw(orc):
    """G = 1 with std > 0: z is increasing in s, so the kept set is the top-B raw scores."""
    rng = np.random.default_rng(9)
    keys, pos, qc, qn, rb = rand_stream(rng, 300, 128, 1, 20000, "bf16")
    _, _, raw = orc.score_stream(keys, pos, 20000, qc, qn, rb, form="fac")
    _, F, _, _ = orc.zmax(raw)
    kept = orc.select(F, 100)
    order = sorted(range(300), key=lambda j: (-raw[0, j], j))[:100]
    assert list(kept) == sorted(order)


def test_p5_positive_scaling_of_statistics(orc):
    """Scaling every qbar and every E|q_f| by c > 0 scales every raw score by c; the z-score
    removes it, so F and the kept set are unchanged."""
    rng = np.random.default_rng(15)
    keys, pos, qc, qn, rb = rand_stream(rng, 400, 128, 4, 9000, "bf16")
    _, _, raw1 = orc.score_stream(keys, pos, 9000, qc, qn, rb, form="fac")
    _, _, raw2 = orc.score_stream(keys, pos, 9000, qc * np.float32(4.0), qn * np.float32(4.0), rb, form="fac")
    np.testing.assert_allclose(raw2, 4.0 * raw1, rtol=1e-13, atol=1e-12)
    _, F1, _, _ = orc.zmax(raw1)
    _, F2, _, _ = orc.zmax(raw2)
    np.testing.assert_allclose(F1, F2, atol=1e-12)
    gap = np.sort(F1)[::-1]
    if gap[99] - gap[100] > 1e-9:
        assert np.array_equal(orc.select(F1, 100), orc.select(F2, 100))


# ---- P9: compaction ------------------------------------------------------------------------------

def test_p9_compaction_is_fancy_indexing(orc):
    rng = np.random.default_rng(19)
    rows = rng.integers(0, 2 ** 16, (50, 128), dtype=np.uint16)
    kept = np.sort(rng.choice(50, 20, replace=False)).astype(np.int32)
    out = orc.compact_rows(rows, kept)
    np.testing.assert_array_equal(out[:20], rows[kept])
    np.testing.assert_array_equal(out[20:], rows[20:])


# ---- whole-stream driver ------------------------------------------------------------------------

def test_prune_streams_matches_per_step_calls(orc):
    cfg = synth.CONFIGS[2]
    wl = synth.make_host(cfg)
    k = wl["k"].reshape(-1, cfg.n_keys, 128)[:3]
    p = wl["pos"].reshape(-1, cfg.n_keys)[:3]
    res = orc.prune_streams(k, p, wl["t"], wl["qc"], wl["qn"], wl["rb"], cfg.budget, cfg.n_kv_heads,
                            stream_ids=[0, 1, 2], form="fac", want_raw=True)
    for i in range(3):
        g = i
        _, _, raw = orc.score_stream(k[i], p[i], int(wl["t"][0]), wl["qc"][0, g * 4:(g + 1) * 4],
                                     wl["qn"][0, g * 4:(g + 1) * 4], wl["rb"][0, g * 4:(g + 1) * 4],
                                     form="fac")
        np.testing.assert_array_equal(res["raw"][i], raw)
        _, F, _, _ = orc.zmax(raw)
        np.testing.assert_array_equal(res["F"][i], F)
        np.testing.assert_array_equal(res["kept"][i], orc.select(F, cfg.budget))


# ---- calibration statistics ---------------------------------------------------------------------

def test_calib_identical_queries_are_fully_concentrated(orc):
    """Every captured query the same: the centre is that query, E|q_f| = |q_f| and R_f = 1."""
    rng = np.random.default_rng(401)
    q0 = rng.standard_normal(128).astype(np.float32)
    q = np.tile(q0, (1, 1, 37, 1))
    qc, qn, r = orc.calib_stats(q)
    np.testing.assert_allclose(qc[0, 0], q0, rtol=1e-15)
    np.testing.assert_allclose(qn[0, 0], np.hypot(q0[:64].astype(np.float64), q0[64:]), rtol=1e-14)
    np.testing.assert_allclose(r[0, 0], 1.0, rtol=1e-14)


def test_calib_unit_phasors_give_mean_resultant_length(orc):
    """Unit-norm bands q_f = exp(i theta_n): E|q_f| = 1 and R_f is the mean resultant length
    |mean_n exp(i theta_n)| of the phases (the unit-phasor definition of concentration,
    chenxutan.com/d/2624 section 2.1), worked here with cmath on a small set."""
    rng = np.random.default_rng(402)
    n = 9
    theta = rng.uniform(-math.pi, math.pi, (n, 64))
    q = np.concatenate([np.cos(theta), np.sin(theta)], axis=1).astype(np.float32)
    qc, qn, r = orc.calib_stats(q[None])
    q64 = q.astype(np.float64)
    for f in (0, 5, 63):
        ph = [complex(q64[k, f], q64[k, f + 64]) for k in range(n)]
        mrl = abs(sum(p / abs(p) for p in ph) / n)
        assert abs(r[0, f] - mrl) < 1e-7          # |q_f| = 1 up to the fp32 rounding of cos/sin
        assert abs(qn[0, f] - 1.0) < 1e-7


def test_calib_symmetric_set_has_zero_centre(orc):
    """Queries in opposite pairs (q and -q): the centre is exactly 0 and so is R."""
    rng = np.random.default_rng(403)
    a = rng.standard_normal((5, 128)).astype(np.float32)
    q = np.concatenate([a, -a])[None, None]
    qc, qn, r = orc.calib_stats(q)
    assert np.all(qc == 0.0) and np.all(r == 0.0)
    np.testing.assert_allclose(qn[0, 0], np.hypot(a[:, :64].astype(np.float64), a[:, 64:]).mean(axis=0),
                               rtol=1e-14)


def test_calib_invariants(orc):
    """0 <= R_f <= 1 (triangle inequality); scaling every query by c > 0 scales the centre and
    the mean norm by c and leaves R unchanged; a zero band has R = 0."""
    rng = np.random.default_rng(404)
    q = (rng.standard_normal((2, 3, 50, 128)) + 0.7).astype(np.float32)
    q[1, 2, :, 7] = 0.0
    q[1, 2, :, 71] = 0.0
    qc, qn, r = orc.calib_stats(q)
    assert np.all(r >= 0.0) and np.all(r <= 1.0 + 1e-15)
    assert r[1, 2, 7] == 0.0 and qn[1, 2, 7] == 0.0
    qc4, qn4, r4 = orc.calib_stats(q * np.float32(4.0))
    np.testing.assert_allclose(qc4, 4.0 * qc, rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(qn4, 4.0 * qn, rtol=1e-14)
    np.testing.assert_allclose(r4, r, rtol=1e-13)


def test_calib_bf16_input_reads_exact_values(orc):
    """bf16 captures are read exactly: the statistics equal those of the same values in fp32."""
    rng = np.random.default_rng(405)
    q32 = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((1, 2, 20, 128)).astype(np.float32)))
    a = orc.calib_stats(synth.f32_to_bf16_bits(q32))
    b = orc.calib_stats(q32)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ---- P12: the R-weighted trigonometric term ------------------------------------------------------

def test_p12_weight_r_limits(orc):
    """R = 1 in every band: the weighted form equals the plain one (no norm term either); R = 0:
    the trigonometric part vanishes and the score is the norm score sum_f E|q_f| |k_f|."""
    rng = np.random.default_rng(120)
    keys, pos, qc, qn, _ = rand_stream(rng, 40, 128, 3, 9000, "bf16")
    ones = np.ones((3, 64), np.float32)
    a = orc.score_stream(keys, pos, 9000, qc, qn, ones, form="fac", weight_r=True)
    b = orc.score_stream(keys, pos, 9000, qc, qn, ones, form="fac")
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    zeros = np.zeros((3, 64), np.float32)
    st, sn, raw = orc.score_stream(keys, pos, 9000, qc, qn, zeros, form="lit", weight_r=True)
    assert np.all(st == 0.0)
    kt = keys_f64(keys)
    mag = np.hypot(kt[:, :64], kt[:, 64:])
    np.testing.assert_allclose(raw, qn.astype(np.float64) @ mag.T, rtol=1e-13)


@pytest.mark.parametrize("form", ["lit", "fac"])
def test_p12_weight_r_single_band_closed_form(orc, form):
    """One band with R_f = 0.3: s = 0.3 |q||k| mean_d cos(w_f (t+d-p) + arg q - arg k)
    + 0.7 E|q_f| |k_f|, worked with cmath."""
    d, t, f = 128, 4000, 11
    w = synth.omega_table(d)
    qc = np.zeros((1, d), np.float32)
    qc[0, f], qc[0, f + 64] = 1.5, -0.25
    post = np.zeros((2, d), np.float32)
    post[:, f] = [0.75, -2.0]
    post[:, f + 64] = [1.25, 0.5]
    pos = np.array([100, 3900], np.int32)
    qn = np.full((1, 64), 2.5, np.float32)
    rb = np.full((1, 64), 0.3, np.float32)
    _, _, raw = orc.score_stream(post, pos, t, qc, qn, rb, form=form, weight_r=True)
    q = complex(1.5, -0.25)
    R = float(np.float32(0.3))
    for j in range(2):
        kt = complex(float(post[j, f]), float(post[j, f + 64]))
        k = kt * complex(math.cos(w[f] * pos[j]), -math.sin(w[f] * pos[j]))
        trig = sum(abs(q) * abs(k) * math.cos(w[f] * (t + dd - int(pos[j])) + math.atan2(q.imag, q.real)
                                              - math.atan2(k.imag, k.real)) for dd in D_DEF) / len(D_DEF)
        val = R * trig + (1 - R) * 2.5 * abs(k)
        assert abs(raw[0, j] - val) < 1e-12 * (abs(q) * abs(k) + 2.5 * abs(k))


# ---- P13: the maximum over the future offsets ----------------------------------------------------

def test_p13_max_over_one_offset_is_the_plain_score(orc):
    """D with a single offset: the maximum and the mean are the same number."""
    rng = np.random.default_rng(130)
    keys, pos, qc, qn, rb = rand_stream(rng, 30, 128, 3, 7000, "bf16")
    for dd in (0, 1, 4096):
        a = orc.score_stream(keys, pos, 7000, qc, qn, rb, offsets=(dd,), form="max")
        b = orc.score_stream(keys, pos, 7000, qc, qn, rb, offsets=(dd,), form="lit")
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_p13_max_is_the_largest_per_offset_rope_dot(orc):
    """The max form equals the largest over d of <RoPE(qbar, t+d), ktilde_j> (numpy fp64 RoPE) when
    the query equals its centre, and it is never below the offset mean."""
    rng = np.random.default_rng(131)
    d, G, N, t = 128, 2, 25, 12000
    keys, pos, qc, qn, rb = rand_stream(rng, N, d, G, t, "f32")
    w = synth.omega_table(d)
    kt = keys_f64(keys)
    st, _, _ = orc.score_stream(keys, pos, t, qc, qn, rb, form="max")
    per = np.stack([np_rope(qc.astype(np.float64), t + dd, w) @ kt.T for dd in D_DEF])
    expect = per.max(axis=0)
    scale = np.abs(np_rope(qc.astype(np.float64), t, w)) @ np.abs(kt).T
    assert np.max(np.abs(st - expect) / scale) < 1e-11
    mean, _, _ = orc.score_stream(keys, pos, t, qc, qn, rb, form="lit")
    assert np.all(st >= mean - 1e-9 * scale)


def test_p13_max_single_band_closed_form(orc):
    """One band: max_d |q||k| cos(w_f (t+d-p) + arg q - arg k) + the norm term, with cmath."""
    d, t, f = 128, 5000, 3
    w = synth.omega_table(d)
    qc = np.zeros((1, d), np.float32)
    qc[0, f], qc[0, f + 64] = -1.0, 0.5
    post = np.zeros((2, d), np.float32)
    post[:, f] = [1.5, -0.25]
    post[:, f + 64] = [0.5, 2.0]
    pos = np.array([7, 4990], np.int32)
    qn = np.full((1, 64), 1.25, np.float32)
    rb = np.full((1, 64), 0.75, np.float32)
    _, _, raw = orc.score_stream(post, pos, t, qc, qn, rb, form="max")
    q = complex(-1.0, 0.5)
    for j in range(2):
        kt = complex(float(post[j, f]), float(post[j, f + 64]))
        k = kt * complex(math.cos(w[f] * pos[j]), -math.sin(w[f] * pos[j]))
        trig = max(abs(q) * abs(k) * math.cos(w[f] * (t + dd - int(pos[j])) + math.atan2(q.imag, q.real)
                                              - math.atan2(k.imag, k.real)) for dd in D_DEF)
        val = trig + (1 - float(np.float32(0.75))) * 1.25 * abs(k)
        assert abs(raw[0, j] - val) < 1e-12 * (abs(q) * abs(k) + abs(k))
