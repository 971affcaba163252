"""GPU parity of the scoring variants that need each key's position (run on an MI355X).

TRIA_PER_KEY_PHASE scores post-RoPE keys in the literal per-key form (phase recovery of every
band, then the distance phase w_f (t - p_j)); TRIA_KEYS_PRE_ROPE scores a cache that keeps keys
before RoPE.  Both run through the C ABI and are compared with the fp64 oracle (its post-RoPE or
pre-RoPE mode) to the same bars as the default path: raw and final scores within 1e-4 relative,
kept sets equal up to near-threshold keys, selection and compaction bit-exact.
"""
import numpy as np
import pytest

import synth
from tests import gpu_check as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_compression_tria_amd as T
    T.lib()
    return T


def test_per_key_phase_config2_literal_oracle(orc, T):
    gc.run_case(orc, T, synth.CONFIGS[2], form="lit", flags=T.PER_KEY_PHASE)


def test_keys_pre_rope_config1_fp32_literal_oracle(orc, T):
    gc.run_case(orc, T, synth.CONFIGS[1], form="lit", flags=T.KEYS_PRE_ROPE)


def test_keys_pre_rope_config2(orc, T):
    gc.run_case(orc, T, synth.CONFIGS[2], flags=T.KEYS_PRE_ROPE)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("flags", [1, 2])
def test_variant_group_sizes(orc, T, G, flags):
    cfg = gc.variant(2, name=f"var{flags}-g{G}", n_q_heads=2 * G, n_kv_heads=2, n_seq=2, n_keys=700, budget=500,
                     t_fixed=9000, calib="uniform_r", r_range=(0.6, 0.99), seed=300 + G)
    gc.run_case(orc, T, cfg, flags=flags)


@pytest.mark.parametrize("G,dtype,N,flags", [(8, "bf16", 5000, 1), (8, "bf16", 5000, 2), (3, "f32", 7000, 1),
                                             (3, "f32", 7000, 3)])
def test_variant_ragged_tiles(orc, T, G, dtype, N, flags):
    """Several 1024-key tiles with a ragged last one; flags 3 (both set) is the pre-RoPE form."""
    cfg = gc.variant(2, name=f"var{flags}-g{G}-{dtype}-N{N}", n_q_heads=G, n_kv_heads=1, n_seq=3, n_keys=N,
                     budget=N // 3 + 7, dtype=dtype, t_fixed=N + 1000, calib="head_r", r_range=(0.6, 0.99),
                     seed=320 + G)
    gc.run_case(orc, T, cfg, flags=flags)


def test_per_key_phase_large_positions(orc, T):
    """Positions up to 9e4: band 0 turns 14000 times; the exact range reduction keeps the phase."""
    cfg = gc.variant(2, name="var1-long", n_q_heads=2, n_kv_heads=1, n_seq=1, n_keys=70001, budget=7000,
                     t_fixed=90000, calib="head_r", r_range=(0.6, 0.99), seed=330)
    gc.run_case(orc, T, cfg, flags=T.PER_KEY_PHASE)


def test_per_key_phase_agrees_with_default_path(T):
    """Same post-RoPE cache scored both ways: final scores agree to 2e-4 relative (both are within
    1e-4 of the oracle), and the kept sets match except at near-ties."""
    import torch
    cfg = gc.variant(5, name="c5-shape-small", n_layers=2, n_seq=1, n_keys=4096, budget=384, t_fixed=4095)
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    F0 = T.score(calib, dev["k"], dev["t_dev"], check=True)
    F1 = T.score(calib, dev["k"], dev["t_dev"], pos=dev["pos"], flags=T.PER_KEY_PHASE, check=True)
    torch.cuda.synchronize()
    a, b = F0.cpu().numpy().astype(np.float64), F1.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(a - b) / np.maximum(np.abs(a), 1.0)) <= 2e-4
    calib.free()


# ---- pre-RoPE keys on the matrix cores (streams long enough for the staged stream clusters) -------

def _pre_rope_workspaces(T, calib, cfg):
    """The matrix-core path stages no raw scores; the vector path (forced by the tiled flag) does."""
    mfma = T.score_workspace_bytes(calib, cfg.n_seq, cfg.n_keys, flags=T.KEYS_PRE_ROPE)
    valu = T.score_workspace_bytes(calib, cfg.n_seq, cfg.n_keys, flags=T.KEYS_PRE_ROPE | T.SCORE_TILED)
    return mfma, valu


def test_pre_rope_matrix_cores_config5_shape(orc, T):
    """Qwen3-32B heads (8 KV heads of 8 queries), 2 layers of one sequence, 32768 pre-RoPE keys per
    stream at positions 0..32767: every stream against the oracle."""
    cfg = gc.variant(5, name="pre-rope-c5-shape", n_layers=2, n_seq=1, seed=370)
    out, _ = gc.run_case(orc, T, cfg, flags=T.KEYS_PRE_ROPE)
    wl = synth.make_host(cfg, pre_rope=True)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    mfma, valu = _pre_rope_workspaces(T, calib, cfg)
    assert mfma < valu // 4, (mfma, valu)
    calib.free()


@pytest.mark.parametrize("G,N,t", [(8, 5000, 2 ** 31 - 1), (4, 9000, 2 ** 31 - 7), (2, 20000, 1_000_003)])
def test_pre_rope_matrix_cores_large_positions(orc, T, G, N, t):
    """Positions drawn up to t (up to 2^31 - 1): the 32-bit turn fractions of every band (signed low
    word, adjusted high word) must match the oracle's exact phases; ragged last tiles."""
    cfg = gc.variant(2, name=f"pre-rope-g{G}-N{N}-t{t}", n_q_heads=2 * G, n_kv_heads=2, n_seq=2, n_keys=N,
                     budget=N // 4 + 3, t_fixed=t, calib="head_r", r_range=(0.6, 0.99), seed=371 + G)
    gc.run_case(orc, T, cfg, flags=T.KEYS_PRE_ROPE)


@pytest.mark.parametrize("G,N,B", [(4, 700, 500), (8, 2176, 2048)])
def test_pre_rope_many_short_streams_on_the_matrix_cores(orc, T, G, N, B):
    """512 pre-RoPE streams that each fit one block take the staged clusters with turned keys (the
    workspace holds no raw scores): every stream against the oracle."""
    cfg = gc.variant(2, name=f"pre-rope-short-g{G}-N{N}", n_layers=32, n_seq=2, n_q_heads=8 * G, n_kv_heads=8,
                     n_keys=N, budget=B, t_fixed=N + 5000, seed=390 + G)
    assert cfg.n_streams == 512
    gc.run_case(orc, T, cfg, flags=T.KEYS_PRE_ROPE)
    wl = synth.make_host(cfg, pre_rope=True)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    mfma, valu = _pre_rope_workspaces(T, calib, cfg)
    assert mfma < valu, (mfma, valu)
    calib.free()


def test_pre_rope_matrix_cores_agree_with_vector_alu(T):
    """The same pre-RoPE cache scored on the matrix cores and on the vector ALU (the tiled flag
    keeps long pre-RoPE streams there): final scores within 2e-4 relative (both are within 1e-4 of
    the oracle), identical kept sets away from near-ties."""
    import torch
    cfg = gc.variant(5, name="pre-rope-c5-2way", n_layers=1, n_seq=1, n_keys=24000, budget=2500, seed=380,
                     positions="gapped", t_fixed=60000)
    wl = synth.make_host(cfg, pre_rope=True)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    mfma, valu = _pre_rope_workspaces(T, calib, cfg)
    assert mfma < valu // 4, (mfma, valu)
    F0 = T.score(calib, dev["k"], dev["t_dev"], pos=dev["pos"], flags=T.KEYS_PRE_ROPE, check=True)
    F1 = T.score(calib, dev["k"], dev["t_dev"], pos=dev["pos"], flags=T.KEYS_PRE_ROPE | T.SCORE_TILED, check=True)
    torch.cuda.synchronize()
    a, b = F0.cpu().numpy().astype(np.float64), F1.cpu().numpy().astype(np.float64)
    err = np.max(np.abs(a - b) / np.maximum(np.abs(a), 1.0))
    print(f"\n[ok] pre-RoPE matrix cores vs vector ALU: F err {err:.2e}", flush=True)
    assert err <= 2e-4
    calib.free()


def test_variant_budget_one_and_single_key(orc, T):
    gc.run_case(orc, T, gc.variant(2, name="var-b1", n_q_heads=8, n_kv_heads=2, n_keys=300, budget=1, seed=341),
                flags=T.KEYS_PRE_ROPE)
    out, _ = gc.run_case(orc, T, gc.variant(2, name="var-bN", n_q_heads=8, n_kv_heads=2, n_keys=300, budget=300,
                                            seed=342), flags=T.PER_KEY_PHASE)
    assert np.array_equal(out["kept"], np.tile(np.arange(300), (2, 1)))
    import torch
    cfg = gc.variant(2, name="var-n1", n_q_heads=4, n_kv_heads=1, n_keys=1, budget=1, t_fixed=5000, seed=343,
                     positions="contiguous")
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], 1)
    for flags in (T.PER_KEY_PHASE, T.KEYS_PRE_ROPE):
        F = T.score(calib, dev["k"], dev["t_dev"], pos=dev["pos"], flags=flags, check=True)
        torch.cuda.synchronize()
        assert F.cpu().numpy().ravel().tolist() == [0.0]
    calib.free()


def test_variant_requires_positions(T):
    """The variants read key positions: a null pos is rejected before any launch."""
    cfg = gc.variant(2, name="var-nopos", n_q_heads=4, n_kv_heads=1, n_keys=64, budget=8, seed=344,
                     positions="contiguous")
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], 1)
    with pytest.raises(T.TriaError):
        T.score(calib, dev["k"], dev["t_dev"], flags=T.PER_KEY_PHASE)
    calib.free()


# ---- R-weighted trigonometric term (TRIA_TRIG_WEIGHT_R) -------------------------------------------

def test_weight_r_config2_literal_oracle(orc, T):
    """Raw scores kept on chip (one block per stream), bf16."""
    gc.run_case(orc, T, synth.CONFIGS[2], form="lit", flags=T.TRIG_WEIGHT_R)


def test_weight_r_config1_fp32(orc, T):
    """fp32 cache: the vector-ALU scorer."""
    gc.run_case(orc, T, synth.CONFIGS[1], form="lit", flags=T.TRIG_WEIGHT_R)


@pytest.mark.parametrize("G,dtype,N", [(8, "bf16", 5000), (3, "f32", 7000), (2, "bf16", 70001)])
def test_weight_r_long_streams(orc, T, G, dtype, N):
    """Long streams: stream clusters (bf16) and the tiled vector path (fp32)."""
    cfg = gc.variant(2, name=f"wr-g{G}-{dtype}-N{N}", n_q_heads=G, n_kv_heads=1, n_seq=2, n_keys=N,
                     budget=N // 3 + 7, dtype=dtype, t_fixed=N + 1000, calib="head_r", r_range=(0.3, 0.99),
                     seed=350 + G)
    gc.run_case(orc, T, cfg, flags=T.TRIG_WEIGHT_R)


def test_weight_r_with_per_key_flags_is_unsupported(T):
    cfg = gc.variant(2, name="wr-unsup", n_q_heads=4, n_kv_heads=1, n_keys=64, budget=8, seed=360,
                     positions="contiguous")
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], 1)
    for extra in (T.PER_KEY_PHASE, T.KEYS_PRE_ROPE):
        with pytest.raises(T.TriaError) as e:
            T.score(calib, dev["k"], dev["t_dev"], pos=dev["pos"], flags=T.TRIG_WEIGHT_R | extra)
        assert e.value.status == T.E_UNSUPPORTED
    calib.free()


# ---- maximum over the future offsets (TRIA_OFFSET_MAX) -------------------------------------------

def test_offset_max_config2(orc, T):
    gc.run_case(orc, T, synth.CONFIGS[2], form="max", flags=T.OFFSET_MAX)


@pytest.mark.parametrize("G", [1, 3, 5, 8])
def test_offset_max_group_sizes(orc, T, G):
    cfg = gc.variant(2, name=f"omax-g{G}", n_q_heads=2 * G, n_kv_heads=2, n_seq=2, n_keys=700, budget=500,
                     t_fixed=9000, calib="uniform_r", r_range=(0.6, 0.99), seed=370 + G)
    gc.run_case(orc, T, cfg, form="max", flags=T.OFFSET_MAX)


@pytest.mark.parametrize("G,N", [(8, 5000), (2, 20000)])
def test_offset_max_chunks_and_ragged_tail(orc, T, G, N):
    """Several 8192-key chunks per stream (N = 20000) and a ragged last tile."""
    cfg = gc.variant(2, name=f"omax-g{G}-N{N}", n_q_heads=G, n_kv_heads=1, n_seq=2, n_keys=N, budget=N // 3 + 7,
                     t_fixed=N + 1000, calib="head_r", r_range=(0.6, 0.99), seed=380 + G)
    gc.run_case(orc, T, cfg, form="max", flags=T.OFFSET_MAX)


def test_offset_max_with_weight_r(orc, T):
    cfg = gc.variant(2, name="omax-wr", n_q_heads=8, n_kv_heads=2, n_seq=2, n_keys=1500, budget=600,
                     t_fixed=3000, calib="head_r", r_range=(0.3, 0.99), seed=390)
    gc.run_case(orc, T, cfg, form="max", flags=T.OFFSET_MAX | T.TRIG_WEIGHT_R)


def test_offset_max_custom_offsets(orc, T):
    """A caller's own offset set (three offsets, one of them 0)."""
    import torch
    cfg = gc.variant(2, name="omax-off", n_q_heads=4, n_kv_heads=1, n_seq=1, n_keys=900, budget=300, t_fixed=5000,
                     seed=391)
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    offs = (0, 5, 1000)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], 1, cfg.theta, offsets=offs)
    raw = torch.empty((1, 1, 4, 900), dtype=torch.float32, device="cuda")
    T.score(calib, dev["k"], dev["t_dev"], raw=raw, flags=T.OFFSET_MAX, check=True)
    torch.cuda.synchronize()
    res = orc.prune_streams(gc.streams_of(wl["k"], 900), gc.streams_of(wl["pos"], 900), wl["t"], wl["qc"], wl["qn"],
                            wl["rb"], 300, 1, offsets=offs, form="max", want_raw=True)
    gc.check_raw(raw.cpu().numpy().reshape(1, 4, 900), res["raw"])
    calib.free()


@pytest.mark.parametrize("n_off", [17, 18, 19, 32])
def test_offset_max_many_offsets(orc, T, n_off):
    """Offset sets of the default size (17), one past it and the largest supported (32): each
    offset's operands take 4 KB of the block's LDS.  Raw and final scores against the oracle."""
    import torch
    G, N = 8, 2500
    cfg = gc.variant(2, name=f"omax-n{n_off}", n_q_heads=G, n_kv_heads=1, n_seq=1, n_keys=N, budget=800,
                     t_fixed=N + 3000, seed=393 + n_off)
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    offs = tuple(sorted((i * 7919) % 50000 for i in range(n_off)))     # distinct, 0 among them
    assert len(set(offs)) == n_off
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], 1, cfg.theta, offsets=offs)
    raw = torch.empty((1, 1, G, N), dtype=torch.float32, device="cuda")
    F = T.score(calib, dev["k"], dev["t_dev"], raw=raw, flags=T.OFFSET_MAX, check=True)
    torch.cuda.synchronize()
    res = orc.prune_streams(gc.streams_of(wl["k"], N), gc.streams_of(wl["pos"], N), wl["t"], wl["qc"], wl["qn"],
                            wl["rb"], cfg.budget, 1, offsets=offs, form="max", want_raw=True)
    e_raw = gc.check_raw(raw.cpu().numpy().reshape(1, G, N), res["raw"])
    e_F = gc.check_F(F.cpu().numpy().reshape(1, N), res["F"])
    print(f"[ok] {n_off} offsets: raw err {e_raw:.2e}  F err {e_F:.2e}", flush=True)
    calib.free()


@pytest.mark.parametrize("variant", ["offset_max", "weight_r", "per_key_phase"])
def test_variants_config5_shape(orc, T, variant):
    """The variants the bench times, at Qwen3-32B stream shapes (8 KV heads of 8 queries, 32768
    keys, B = 3072): every stream of one sequence against the oracle, one layer for the maximum over
    the offsets (its oracle evaluates all 17 offsets per key and head), two for the others."""
    flags = {"offset_max": T.OFFSET_MAX, "weight_r": T.TRIG_WEIGHT_R, "per_key_phase": T.PER_KEY_PHASE}[variant]
    cfg = gc.variant(5, name=f"{variant}-c5-shape", n_layers=1 if variant == "offset_max" else 2, n_seq=1,
                     seed=396)
    gc.run_case(orc, T, cfg, form="max" if variant == "offset_max" else "fac", flags=flags)


def test_offset_max_unsupported_cases(T):
    cfg = gc.variant(1, name="omax-f32", n_keys=256, budget=64, seed=392, positions="contiguous", t_fixed=300)
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    with pytest.raises(T.TriaError) as e:                      # fp32 cache
        T.score(calib, dev["k"], dev["t_dev"], flags=T.OFFSET_MAX)
    assert e.value.status == T.E_UNSUPPORTED
    with pytest.raises(T.TriaError) as e:                      # with a per-key flag
        T.score(calib, dev["k"], dev["t_dev"], pos=dev["pos"], flags=T.OFFSET_MAX | T.PER_KEY_PHASE)
    assert e.value.status == T.E_UNSUPPORTED
    calib.free()
