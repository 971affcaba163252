"""GPU parity: the HIP path through the C ABI against the fp64 oracle (run on an MI355X).

Covers the small configurations in full, group sizes 1..8, both scoring paths (raw scores kept
on chip, and the tiled path with a ragged last tile), fp32 and bf16 caches, and the degenerate
cases (one key, B >= N, constant streams, ties, non-finite keys).
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


variant = gc.variant
run_case = gc.run_case


def test_config1_tiny_fp32_literal_oracle(orc, T):
    run_case(orc, T, synth.CONFIGS[1], form="lit")


def test_config2_qwen3_8b_layer_literal_oracle(orc, T):
    run_case(orc, T, synth.CONFIGS[2], form="lit")


@pytest.mark.parametrize("G", [1, 2, 3, 5, 6, 7, 8])
def test_group_sizes(orc, T, G):
    cfg = variant(2, name=f"g{G}", n_q_heads=2 * G, n_kv_heads=2, n_seq=2, n_keys=700, budget=500,
                  t_fixed=9000, calib="uniform_r", r_range=(0.6, 0.99), seed=100 + G)
    run_case(orc, T, cfg)


@pytest.fixture(params=["auto", "tiled"])
def path(request):
    """Long bf16 streams: the stream-cluster path (auto) and the tiled path (TRIA_SCORE_TILED)."""
    return request.param


def path_flags(T, path):
    return T.SCORE_TILED if path == "tiled" else 0


@pytest.mark.parametrize("G,dtype,N", [(8, "bf16", 5000), (4, "bf16", 5000), (3, "f32", 7000), (1, "bf16", 21000)])
def test_tiled_path_ragged_tail(orc, T, path, G, dtype, N):
    cfg = variant(2, name=f"tiled-g{G}-{dtype}-N{N}-{path}", n_q_heads=G, n_kv_heads=1, n_seq=3, n_keys=N,
                  budget=N // 3 + 7, dtype=dtype, t_fixed=N + 1000, calib="head_r", r_range=(0.6, 0.99),
                  seed=200 + G)
    run_case(orc, T, cfg, flags=path_flags(T, path))


def test_tiled_path_long_stream(orc, T, path):
    """A stream of 70001 keys: 69 tiles of 1024 keys, the last one ragged (369 keys); on the
    staged cluster path (G = 2) 16 blocks of 4384 keys, the last one with 4241."""
    cfg = variant(2, name=f"tiled-long-{path}", n_q_heads=2, n_kv_heads=1, n_seq=1, n_keys=70001, budget=7000,
                  t_fixed=90000, calib="head_r", r_range=(0.6, 0.99), seed=210)
    run_case(orc, T, cfg, flags=path_flags(T, path))


def test_cluster_path_many_rounds(orc, T, path):
    """480 streams of 3000 keys with G = 8: on the staged cluster path two blocks per stream
    (1504 and 1496 keys), 128 clusters per grid, so streams run up to four rounds; sampled
    streams on both sides of every round boundary."""
    cfg = variant(2, name=f"rounds-{path}", n_q_heads=64, n_kv_heads=8, n_seq=1, n_layers=60, n_keys=3000,
                  budget=900, t_fixed=4000, calib="head_r", r_range=(0.6, 0.99), seed=212)
    run_case(orc, T, cfg, sample=np.array([0, 1, 127, 128, 255, 256, 383, 384, 479]), flags=path_flags(T, path))


def test_staged_parts_rotate_with_a_ragged_last_part(orc, T):
    """G = 8 and 32760 keys: 16 blocks of 2048 keys per stream, the last with 2040, all with 16
    tiles per wave, so blocks take a different part in every round; 40 streams over 16 clusters
    give two or three rounds.  Sampled streams on both sides of the round boundaries."""
    cfg = variant(2, name="g8-N32760-rotate", n_q_heads=8, n_kv_heads=1, n_seq=1, n_layers=40, n_keys=32760,
                  budget=3000, t_fixed=33000, calib="head_r", r_range=(0.6, 0.99), seed=215)
    run_case(orc, T, cfg, sample=np.array([0, 7, 15, 16, 23, 31, 32, 39]))


@pytest.mark.parametrize("N", [30000, 32768])
def test_staged_g4_long_rounds(orc, T, N):
    """G = 4: 8 blocks per stream.  30000 keys give 30 tiles per wave and round (not every part
    full: fixed parts); 32768 keys give 32 (every part full: parts rotate).  Both defer 16 tiles
    and fetch the cluster's partials during them; 40 streams over 32 clusters give two rounds."""
    cfg = variant(2, name=f"g4-N{N}-rounds", n_q_heads=4, n_kv_heads=1, n_seq=1, n_layers=40, n_keys=N,
                  budget=N // 10, t_fixed=N + 500, calib="head_r", r_range=(0.6, 0.99), seed=216)
    run_case(orc, T, cfg, sample=np.array([0, 8, 31, 32, 39]))


@pytest.mark.parametrize("N", [65536, 100001])
def test_widest_clusters(orc, T, N):
    """G = 8: 65536 keys fill the staged path's widest cluster (32 blocks of 2048 keys); 100001
    keys are past its reach and run on the register-ring cluster path (32 blocks of 3136 keys,
    the last one with 2785)."""
    cfg = variant(2, name=f"g8-N{N}", n_q_heads=8, n_kv_heads=1, n_seq=2, n_keys=N, budget=N // 11,
                  t_fixed=N + 5000, calib="head_r", r_range=(0.6, 0.99), seed=214)
    run_case(orc, T, cfg)


def test_stream_beyond_cluster_reach(orc, T):
    """G = 8 and 140000 keys need more than 32 blocks of on-chip raw scores: the tiled path
    takes over by itself."""
    cfg = variant(2, name="g8-N140000", n_q_heads=8, n_kv_heads=1, n_seq=1, n_keys=140000, budget=9000,
                  t_fixed=150000, calib="head_r", r_range=(0.6, 0.99), seed=213)
    run_case(orc, T, cfg)


def test_cluster_and_tiled_paths_agree(T):
    """Same cache scored on both long-stream paths: final scores within 2e-6 relative (both
    are fp32 scores of the same matrix-core products; only the summation order of the
    statistics differs)."""
    import torch
    cfg = variant(5, name="c5-shape-2layer", n_layers=2, n_seq=1, n_keys=32768, budget=3072, t_fixed=32767)
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    F0 = T.score(calib, dev["k"], dev["t_dev"], flags=T.SCORE_TILED, check=True)
    F1 = T.score(calib, dev["k"], dev["t_dev"], check=True)
    torch.cuda.synchronize()
    a, b = F0.cpu().numpy().astype(np.float64), F1.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(a - b) / np.maximum(np.abs(a), 1.0)) <= 2e-6
    calib.free()


def test_tiled_path_many_streams_ragged_tail(orc, T):
    """40 streams of 65236 keys (63 * 1024 + 724): every stream ends in a ragged tile."""
    cfg = variant(2, name="tiled-many", n_q_heads=16, n_kv_heads=8, n_seq=5, n_layers=1, n_keys=65236,
                  budget=6000, t_fixed=70000, calib="head_r", r_range=(0.6, 0.99), seed=211)
    rng = np.random.default_rng(211)
    run_case(orc, T, cfg, sample=np.sort(rng.choice(cfg.n_streams, 5, replace=False)))


def test_contiguous_positions_config5_shape_small(orc, T):
    cfg = variant(5, name="c5-shape-small", n_layers=2, n_seq=1, n_keys=4096, budget=384, t_fixed=4095)
    run_case(orc, T, cfg)


def test_budget_one_and_budget_at_least_n(orc, T):
    run_case(orc, T, variant(2, name="b1", n_q_heads=8, n_kv_heads=2, n_keys=300, budget=1, seed=31))
    out, _ = run_case(orc, T, variant(2, name="bN", n_q_heads=8, n_kv_heads=2, n_keys=300, budget=300, seed=32))
    assert np.array_equal(out["kept"], np.tile(np.arange(300), (2, 1)))
    out, _ = run_case(orc, T, variant(2, name="bbig", n_q_heads=8, n_kv_heads=2, n_keys=300, budget=5000, seed=33))
    assert np.array_equal(out["kept"], np.tile(np.arange(300), (2, 1)))


def test_single_key_stream(orc, T):
    out, _ = run_case(orc, T, variant(2, name="n1", n_q_heads=4, n_kv_heads=1, n_keys=129, budget=1, seed=34))
    import torch
    # one key: its std is zero, z = 0
    cfg = variant(2, name="n1-exact", n_q_heads=4, n_kv_heads=1, n_keys=1, budget=1, t_fixed=5000, seed=35,
                  positions="contiguous")
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], 1)
    F = T.score(calib, dev["k"], dev["t_dev"], check=True)
    kept = T.select_topB(F, 1)
    torch.cuda.synchronize()
    assert F.cpu().numpy().ravel().tolist() == [0.0]
    assert kept.cpu().numpy().ravel().tolist() == [0]


def _constant_stream_workload(N=500, B=300):
    cfg = variant(2, name="const", n_q_heads=4, n_kv_heads=2, n_keys=N, budget=B, seed=36)
    wl = synth.make_host(cfg)
    k = wl["k"].copy()
    k[0, 0, 0, :, :] = k[0, 0, 0, 0, :]      # every key of stream 0 identical
    wl["k"] = k
    return cfg, wl


def test_constant_stream_scores_zero_and_keeps_prefix(orc, T):
    import torch
    cfg, wl = _constant_stream_workload()
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads)
    F = T.score(calib, dev["k"], dev["t_dev"], check=True)
    kept = T.select_topB(F, cfg.budget)
    torch.cuda.synchronize()
    F0 = F.cpu().numpy().reshape(2, -1)[0]
    assert np.all(F0 == 0.0)
    assert np.array_equal(kept.cpu().numpy()[0], np.arange(cfg.budget))
    res = orc.prune_streams(gc.streams_of(wl["k"], cfg.n_keys)[:1], gc.streams_of(wl["pos"], cfg.n_keys)[:1],
                            wl["t"], wl["qc"], wl["qn"], wl["rb"], cfg.budget, cfg.n_kv_heads, stream_ids=[0])
    assert np.all(res["F"] == 0.0) and np.array_equal(res["kept"][0], np.arange(cfg.budget))


def test_ties_resolved_to_lower_index(orc, T):
    """Duplicated keys give exactly equal final scores; the selection must take the lower index
    among equal scores (checked bit-exactly against a full sort of the GPU's own scores)."""
    import torch
    cfg = variant(2, name="ties", n_q_heads=8, n_kv_heads=2, n_keys=640, budget=200, seed=37)
    wl = synth.make_host(cfg)
    k = wl["k"].copy()
    k[0, 0, :, 320:, :] = k[0, 0, :, :320, :]          # second half repeats the first half
    wl["k"] = k
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads)
    F = T.score(calib, dev["k"], dev["t_dev"], check=True)
    kept = T.select_topB(F, cfg.budget)
    torch.cuda.synchronize()
    Fh = F.cpu().numpy().reshape(2, -1)
    gc.check_select_exact(orc, kept.cpu().numpy(), Fh, cfg.budget)
    assert np.array_equal(Fh[:, 320:], Fh[:, :320])


def test_nonfinite_key_is_reported(T):
    import torch
    cfg = variant(2, name="nan", n_q_heads=4, n_kv_heads=1, n_keys=256, budget=100, seed=38)
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    dev["k"][0, 0, 0, 17, 5] = float("nan")
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], 1)
    with pytest.raises(T.TriaError) as e:
        T.score(calib, dev["k"], dev["t_dev"], check=True)
    assert e.value.status == T.E_NONFINITE
    # a clean call on the same workspace clears the flag
    dev2 = synth.to_device(wl)
    T.score(calib, dev2["k"], dev2["t_dev"], check=True)
    torch.cuda.synchronize()


def test_scores_are_deterministic(T):
    import torch
    for cfg in (variant(2, name="det", n_seq=1), variant(2, name="det-tiled", n_q_heads=8, n_kv_heads=1,
                                                         n_keys=9000, budget=900, t_fixed=12000)):
        wl = synth.make_host(cfg)
        dev = synth.to_device(wl)
        calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads)
        F1 = T.score(calib, dev["k"], dev["t_dev"], check=True).cpu().numpy()
        F2 = T.score(calib, dev["k"], dev["t_dev"], check=True).cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(F1.view(np.uint32), F2.view(np.uint32))


@pytest.mark.parametrize("G,N,B", [(4, 17, 9), (4, 33, 20), (8, 100, 37), (4, 700, 500), (8, 700, 699)])
def test_many_short_streams_on_the_staged_clusters(orc, T, G, N, B):
    """512 streams that each fit one block take the staged stream clusters (256 or more streams),
    with parts down to one 16-key tile per round and waves without a tile: every stream against
    the oracle (raw and final scores, kept sets, selection, compaction)."""
    pos_mode = "gapped" if N >= 256 else "contiguous"     # gapped draws keep the last 128 recent
    cfg = variant(2, name=f"short-g{G}-N{N}", n_layers=32, n_seq=2, n_q_heads=8 * G, n_kv_heads=8,
                  n_keys=N, budget=B, t_fixed=N + 3000, seed=400 + N + G, positions=pos_mode)
    assert cfg.n_streams == 512
    run_case(orc, T, cfg)
    wl = synth.make_host(cfg)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    # the cluster exchange (2 x 1024 blocks x 8 heads x 4 doubles) is reserved: the staged path
    # was planned; eight streams of the same length stay on chip and reserve none of it
    assert T.score_workspace_bytes(calib, cfg.n_seq, N) > 512 * 1024
    calib.free()
    cfg8 = variant(2, name=f"short8-g{G}-N{N}", n_layers=1, n_seq=1, n_q_heads=8 * G, n_kv_heads=8,
                   n_keys=N, budget=B, t_fixed=N + 3000, seed=401 + N + G, positions=pos_mode)
    wl8 = synth.make_host(cfg8)
    calib8 = T.load_calib(wl8["qc"], wl8["qn"], wl8["rb"], cfg8.n_kv_heads, cfg8.theta)
    assert T.score_workspace_bytes(calib8, 1, N) < 512 * 1024
    calib8.free()


def test_many_single_key_streams_on_the_staged_clusters(T):
    """512 one-key streams (staged clusters, one 16-key tile holding one key per part): every
    head's spread is zero, so every final score is exactly 0, every stream keeps its key, and
    the rows stay where they are."""
    import torch
    cfg = variant(2, name="single-512", n_layers=32, n_seq=2, n_q_heads=32, n_kv_heads=8, n_keys=1, budget=1,
                  t_fixed=5000, seed=420, positions="contiguous")
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    k_before = dev["k"].clone()
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    F, kept = T.prune(calib, dev["k"], dev["v"], dev["pos"], dev["t_dev"], 1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(F).item() == 0 and F.numel() == 512
    assert torch.count_nonzero(kept).item() == 0 and kept.numel() == 512
    assert torch.equal(dev["k"], k_before)
    calib.free()


def test_config5_default_workspace_is_small(T):
    """The prune step's workspace at Qwen3-32B (64 layers, 8 KV heads of 8 queries), 8 sequences
    of 32768 bf16 keys: the default path reserves the matrix-core operands, pivots, the cluster
    exchange and the side sample only (about 68 MB), not the raw scores that only the tiled path
    stages (4.3 GB)."""
    cfg = synth.CONFIGS[5]
    Hq, L = cfg.n_q_heads, cfg.n_layers
    rng = np.random.default_rng(5)
    calib = T.load_calib(rng.standard_normal((L, Hq, 128), dtype=np.float32),
                         np.ones((L, Hq, 64), np.float32), np.full((L, Hq, 64), 0.5, np.float32), cfg.n_kv_heads)
    ws = T.prune_workspace_bytes(calib, cfg.n_seq, cfg.n_keys, cfg.budget)
    assert 0 < ws < 100_000_000, ws
    raw = cfg.n_seq * L * Hq * cfg.n_keys * 4
    assert T.prune_workspace_bytes(calib, cfg.n_seq, cfg.n_keys, cfg.budget, flags=T.SCORE_TILED) > raw


def test_prune_entry_point_matches_separate_calls(T):
    import torch
    cfg = variant(2, name="prune", n_seq=2, seed=39)
    wl = synth.make_host(cfg)
    d1, d2 = synth.to_device(wl), synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads)
    F1 = T.score(calib, d1["k"], d1["t_dev"], check=True)
    kept1 = T.select_topB(F1, cfg.budget)
    T.compact(d1["k"], d1["v"], d1["pos"], kept1, cfg.budget)
    F2, kept2 = T.prune(calib, d2["k"], d2["v"], d2["pos"], d2["t_dev"], cfg.budget)
    torch.cuda.synchronize()
    assert torch.equal(F1, F2) and torch.equal(kept1, kept2)
    assert torch.equal(d1["k"], d2["k"]) and torch.equal(d1["v"], d2["v"]) and torch.equal(d1["pos"], d2["pos"])


@pytest.mark.parametrize("dtype,G,N,B", [("bf16", 4, 5000, 1673), ("f32", 2, 3001, 1000), ("bf16", 8, 32768, 3072),
                                          ("bf16", 4, 9000, 4096), ("bf16", 4, 700, 1), ("bf16", 2, 1025, 1024)])
def test_prune_matches_separate_calls_shapes(T, dtype, G, N, B):
    """tria_prune's F, kept indices and compacted K, V, positions equal those of the three
    separate calls bit for bit, across on-chip, cluster and fp32 shapes and ragged sizes."""
    import torch
    print(f"\n[case] prune vs separate {dtype} G={G} N={N} B={B}", flush=True)
    n_layers = 2 if N > 20000 else 1
    cfg = variant(2, name=f"prune-{dtype}-N{N}", n_q_heads=2 * G, n_kv_heads=2, n_seq=2, n_layers=n_layers,
                  n_keys=N, budget=B, dtype=dtype, t_fixed=N + 500, calib="head_r", r_range=(0.6, 0.99),
                  seed=40 + G)
    wl = synth.make_host(cfg)
    d1, d2 = synth.to_device(wl), synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    F1 = T.score(calib, d1["k"], d1["t_dev"], check=True)
    kept1 = T.select_topB(F1, B)
    T.compact(d1["k"], d1["v"], d1["pos"], kept1, B)
    F2, kept2 = T.prune(calib, d2["k"], d2["v"], d2["pos"], d2["t_dev"], B)
    torch.cuda.synchronize()
    assert torch.equal(F1, F2) and torch.equal(kept1, kept2)
    assert torch.equal(d1["k"], d2["k"]) and torch.equal(d1["v"], d2["v"]) and torch.equal(d1["pos"], d2["pos"])
    calib.free()


@pytest.mark.parametrize("N", [700, 20000, 40000])
def test_prune_after_a_failed_score_keeps_every_row(T, N):
    """A non-finite key makes the score fail on the device; tria_prune cannot return that (it is
    asynchronous), so its selection reads the score's error word and keeps every row in place:
    kept = 0..B-1 and K, V and positions unchanged; the check then reports the failure.  N covers
    the three selection kernels (LDS copy, registers, global passes)."""
    import torch
    print(f"\n[case] prune after a failed score N={N}", flush=True)
    cfg = variant(2, name=f"guard-N{N}", n_q_heads=8, n_kv_heads=2, n_seq=1, n_keys=N, budget=N // 3,
                  t_fixed=N + 100, calib="head_r", r_range=(0.6, 0.99), seed=61)
    wl = synth.make_host(cfg)
    dev = synth.to_device(wl)
    dev["k"][0, 0, 1, N // 2, 7] = float("inf")
    k0, v0, p0 = dev["k"].clone(), dev["v"].clone(), dev["pos"].clone()
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    B = cfg.budget
    kept = torch.full((cfg.n_streams, B), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(T.TriaError) as e:
        T.prune(calib, dev["k"], dev["v"], dev["pos"], dev["t_dev"], B, kept=kept)
    assert e.value.status == T.E_NONFINITE
    torch.cuda.synchronize()
    ar = torch.arange(B, dtype=torch.int32, device="cuda").expand(cfg.n_streams, B)
    assert torch.equal(kept, ar)
    assert torch.equal(dev["k"].view(torch.int16), k0.view(torch.int16))
    assert torch.equal(dev["v"], v0) and torch.equal(dev["pos"], p0)
    calib.free()


@pytest.mark.parametrize("N,G", [(2176, 4), (9000, 8)])
def test_prune_step_replays_in_a_hip_graph(T, N, G):
    """The whole step captured once in a HIP graph (torch.cuda.graph) and replayed several times,
    with eager work and synchronisations between replays: every replay's F, kept indices and
    compacted cache equal an eager run's bit for bit (on-chip path N = 2176, stream clusters
    N = 9000, G = 8)."""
    import torch
    print(f"\n[case] graph replay N={N} G={G}", flush=True)
    cfg = variant(2, name=f"graph-N{N}", n_q_heads=2 * G, n_kv_heads=2, n_seq=2, n_keys=N, budget=N // 4,
                  t_fixed=N + 100, calib="head_r", r_range=(0.6, 0.99), seed=50 + G)
    wl = synth.make_host(cfg)
    ref = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    B = cfg.budget
    F_ref, kept_ref = T.prune(calib, ref["k"], ref["v"], ref["pos"], ref["t_dev"], B)
    torch.cuda.synchronize()
    dev = synth.to_device(wl)
    k0, v0, p0 = dev["k"].clone(), dev["v"].clone(), dev["pos"].clone()
    S, L, Hkv = dev["k"].shape[:3]
    F = torch.empty((S, L, Hkv, N), dtype=torch.float32, device="cuda")
    kept = torch.empty((S * L * Hkv, B), dtype=torch.int32, device="cuda")
    ws = T.workspace(T.prune_workspace_bytes(calib, S, N, B, dev["k"].dtype))
    T.prune(calib, dev["k"], dev["v"], dev["pos"], dev["t_dev"], B, F=F, kept=kept, ws=ws)   # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        # no check inside the capture (it synchronises); the workspace is checked after each replay
        T.prune(calib, dev["k"], dev["v"], dev["pos"], dev["t_dev"], B, F=F, kept=kept, ws=ws, check=False)
    for rep in range(3):
        dev["k"].copy_(k0)
        dev["v"].copy_(v0)
        dev["pos"].copy_(p0)
        F.zero_()
        kept.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        T.score_check(ws)
        assert torch.equal(F, F_ref) and torch.equal(kept, kept_ref), f"replay {rep}"
        assert torch.equal(dev["k"], ref["k"]) and torch.equal(dev["v"], ref["v"]) and torch.equal(dev["pos"], ref["pos"])
    calib.free()
