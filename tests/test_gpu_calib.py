"""GPU parity of the calibration-statistics kernel (tria_calib_stats) against the fp64 oracle.

The captured pre-RoPE queries are synthetic: per (layer, head) a centre c = 8 u / |u| plus
N(0, s^2) noise with s drawn per head, so R spans concentrated and diffuse heads.  Bars: centre
within 1e-6 * E|q_f| (an fp64 mean rounded to fp32), E|q_f| within 1e-6 relative, R within
1e-6 absolute; a zero band gives R = 0 exactly; repeated calls give identical bits.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_compression_tria_amd as T
    T.lib()
    return T


def captured_queries(seed, L, Hq, n_cal, dtype):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((L, Hq, 1, 128))
    centre = 8.0 * u / np.linalg.norm(u, axis=-1, keepdims=True)
    spread = rng.uniform(0.05, 3.0, (L, Hq, 1, 1))
    q = (centre + spread * rng.standard_normal((L, Hq, n_cal, 128))).astype(np.float32)
    return q if dtype == "f32" else synth.f32_to_bf16_bits(q)


def to_dev(q):
    import torch
    if q.dtype == np.uint16:
        return torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(q).cuda()


def check(T, orc, q):
    import torch
    qc, qn, rb = T.calib_stats(to_dev(q))
    torch.cuda.synchronize()
    e_qc, e_qn, e_r = orc.calib_stats(q)
    g_qc, g_qn, g_r = (x.cpu().numpy().astype(np.float64) for x in (qc, qn, rb))
    scale = np.concatenate([e_qn, e_qn], axis=-1)
    assert np.all(np.abs(g_qc - e_qc) <= 1e-6 * scale + 1e-30)
    np.testing.assert_allclose(g_qn, e_qn, rtol=1e-6, atol=1e-30)
    assert np.max(np.abs(g_r - e_r)) <= 1e-6
    return g_r, e_r


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_cal", [1, 3, 16, 37, 1000, 4099])
def test_calib_stats_matches_oracle(T, orc, dtype, n_cal):
    print(f"\n[case] calib {dtype} n_cal={n_cal}", flush=True)
    q = captured_queries(500 + n_cal, 2, 3, n_cal, dtype)
    check(T, orc, q)


def test_calib_stats_qwen3_8b_layer(T, orc):
    """One layer of Qwen3-8B shapes (32 query heads) with 4096 captured queries in bf16."""
    print("\n[case] calib qwen3-8b layer", flush=True)
    q = captured_queries(510, 1, 32, 4096, "bf16")
    g_r, _ = check(T, orc, q)
    assert g_r.min() < 0.5 < g_r.max()        # both diffuse and concentrated heads are covered


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_calib_stats_qwen3_32b_head_count(T, orc, dtype):
    """Qwen3-32B's 64 layers x 64 query heads: more heads than resident multi-wave blocks, so one
    wave per head (the launch the calibration bench times), with 43 captured queries (groups of
    eight rows and a ragged tail of three)."""
    print(f"\n[case] calib qwen3-32b head count {dtype}", flush=True)
    q = captured_queries(520, 64, 64, 43, dtype)
    check(T, orc, q)


def test_calib_stats_degenerate_bands(T, orc):
    """A band that is zero in every query has E|q_f| = 0 and R = 0; identical queries give R = 1
    within fp32 rounding."""
    print("\n[case] calib degenerate", flush=True)
    q = captured_queries(511, 1, 2, 40, "f32")
    q[0, 0, :, 5] = 0.0
    q[0, 0, :, 69] = 0.0
    q[0, 1] = q[0, 1, :1]
    g_r, _ = check(T, orc, q)
    assert g_r[0, 0, 5] == 0.0
    np.testing.assert_allclose(g_r[0, 1], 1.0, atol=1e-6)


def test_calib_stats_deterministic_and_feeds_load_calib(T, orc):
    import torch
    q = to_dev(captured_queries(512, 2, 4, 300, "bf16"))
    a = T.calib_stats(q)
    b = T.calib_stats(q)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    calib = T.load_calib(a[0].cpu().numpy(), a[1].cpu().numpy(), a[2].cpu().numpy(), 2)
    calib.free()


def test_calib_stats_rejects_bad_arguments(T):
    import torch
    q = torch.zeros((1, 1, 4, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(T.TriaError):
        T.calib_stats(q)          # head_dim 64
