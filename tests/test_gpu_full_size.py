"""GPU parity at the full sizes of the large workloads, in the launch the benchmark times
(tria_prune over every stream, no raw-score output):

  config 3 (Qwen3-8B, 36 layers, 288 streams of 3200 keys)  every stream against the oracle:
      final scores, kept sets, selection, compaction of K, V and positions; raw scores of every
      stream from a second tria_score call with the raw output;
  config 4 (Qwen3-8B, batch 64, 18432 streams of 2176 keys)  every stream, the same checks
      (raw scores on a seeded sample);
  config 5 (Qwen3-32B, 4096 streams of 32768 keys)  every stream's final scores and kept set
      against the exchange-free tiled path (TRIA_SCORE_TILED), every stream's selection checked
      for the top-B order rule, and 256 seeded streams -- all 16 stream clusters, first, middle
      and last rounds -- against the oracle (raw and final scores, kept sets, selection, a
      bit-exact gather of K, V and positions).

What each stream must satisfy: the top-B of the z-scored, group-maxed scores, in index order
(chenxutan.com/d/2624 section 4.2, prune_kv_cache: top-k, then sort; watermelonwater.tech
"TriAttention 方案设计" item 4: z-score, then the maximum over the GQA group).
"""
import numpy as np
import pytest

import synth
from tests import gpu_check as gc

pytestmark = pytest.mark.gpu

# The tiled path and the stream clusters compute the same fp32 scores from the same matrix-core
# products; only the order in which the per-head sums are added differs.
PATH_RTOL = 2e-6


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import kv_cache_compression_tria_amd as T
    T.lib()
    return T


def select_order_ok(F, kept, B):
    """Vectorised check of the selection rule on every stream: B distinct ascending indices; every
    kept score >= every dropped score; among scores equal to the smallest kept one, the kept keys
    are the lowest indices.  F [n][N] float32 (-0 compares equal to +0), kept [n][B]."""
    n, N = F.shape
    assert kept.shape == (n, B)
    assert np.all(np.diff(kept, axis=1) > 0) and kept.min() >= 0 and kept.max() < N
    Fk = np.take_along_axis(F, kept, axis=1)
    mask = np.zeros((n, N), dtype=bool)
    np.put_along_axis(mask, kept, True, axis=1)
    t = Fk.min(axis=1)
    dropped_max = np.where(mask, -np.inf, F).max(axis=1)
    assert np.all(dropped_max <= t), "a dropped key scores above a kept one"
    # ties at the threshold: no dropped key equal to it may precede a kept key equal to it
    eq = F == t[:, None]
    last_kept_eq = np.where(eq & mask, np.arange(N)[None, :], -1).max(axis=1)
    first_dropped_eq = np.where(eq & ~mask, np.arange(N)[None, :], N).min(axis=1)
    assert np.all(first_dropped_eq > last_kept_eq), "a tie at the threshold went to a higher index"


def oracle_check_streams(orc, T, cfg, wl, ids, kb, vb, pb, out, ka, va, pa, raw=None):
    """Oracle on streams ids (host copies kb, vb, pb taken before the prune); out: GPU F, kept
    (all streams); ka, va, pa: the GPU's compacted rows of the same streams; raw: the GPU's raw
    scores of the same streams [n][G][N] or None."""
    B = cfg.budget
    res = orc.prune_streams(kb, pb, wl["t"], wl["qc"], wl["qn"], wl["rb"], B, cfg.n_kv_heads, stream_ids=ids,
                            form="fac", want_raw=raw is not None)
    e_F = gc.check_F(out["F"][ids], res["F"])
    n_diff = gc.check_kept_sets(out["kept"][ids], res["kept"], res["F"], B)
    gc.check_select_exact(orc, out["kept"][ids], out["F"][ids], B)
    gc.check_compaction(kb, ka, out["kept"][ids], B)
    gc.check_compaction(vb, va, out["kept"][ids], B)
    gc.check_compaction(pb, pa, out["kept"][ids], B)
    e_raw = gc.check_raw(raw, res["raw"]) if raw is not None else None
    return e_F, n_diff, e_raw


def prune_all(T, calib, wl, B):
    """The benchmark's call: tria_prune over every stream (default flags, no raw output)."""
    import torch
    k, v, pos, t = wl["k"], wl["v"], wl["pos"], wl["t_dev"]
    S, L, Hkv, N, _ = k.shape
    ws = T.workspace(T.prune_workspace_bytes(calib, S, N, B, k.dtype))
    F, kept = T.prune(calib, k, v, pos, t, B, ws=ws)
    torch.cuda.synchronize()
    return F, kept


def raw_scores(T, calib, k, t, S, N):
    """tria_score with the raw-score output (same kernels, plus raw stores)."""
    import torch
    L, Hkv = k.shape[1], k.shape[2]
    raw = torch.empty((S, L, calib.n_q_heads, N), dtype=torch.float32, device=k.device)
    F = T.score(calib, k, t, raw=raw, check=True)
    torch.cuda.synchronize()
    return F, raw


def report(capsys, msg):
    """Counts of checked streams go to the terminal even when pytest captures output."""
    with capsys.disabled():
        print(msg, flush=True)


def test_config3_every_stream(orc, T, capsys):
    import torch
    cfg = synth.CONFIGS[3]
    print(f"\n[case] every stream: {cfg.describe()}", flush=True)
    wl_h = synth.make_host(cfg)
    wl = synth.to_device(wl_h)
    N, B, G = cfg.n_keys, cfg.budget, cfg.G
    calib = T.load_calib(wl_h["qc"], wl_h["qn"], wl_h["rb"], cfg.n_kv_heads, cfg.theta)
    F_raw, raw = raw_scores(T, calib, wl["k"], wl["t_dev"], cfg.n_seq, N)
    F, kept = prune_all(T, calib, wl, B)
    assert torch.equal(F, F_raw), "final scores differ between the prune and the raw-output score calls"
    out = {"F": F.cpu().numpy().reshape(-1, N), "kept": kept.cpu().numpy()}
    ids = np.arange(cfg.n_streams)
    kb, vb, pb = (gc.streams_of(wl_h[x], N) for x in ("k", "v", "pos"))
    ka = gc.streams_of(gc.host_cache(wl["k"]), N)
    va = gc.streams_of(gc.host_cache(wl["v"]), N)
    pa = gc.streams_of(wl["pos"].cpu().numpy(), N)
    e_F, n_diff, e_raw = oracle_check_streams(orc, T, cfg, wl_h, ids, kb, vb, pb, out, ka, va, pa,
                                              raw=raw.cpu().numpy().reshape(-1, G, N))
    report(capsys, f"[ok] {len(ids)} of {cfg.n_streams} streams against the oracle: raw err {e_raw:.2e}, F err {e_F:.2e}, "
          f"near-threshold set differences in {n_diff} streams")
    calib.free()


@pytest.fixture(scope="module")
def config4(T):
    """Config 4 on the device, pruned once by tria_prune; host copies of the inputs and outputs."""
    import torch
    cfg = synth.CONFIGS[4]
    print(f"\n[setup] every stream: {cfg.describe()}", flush=True)
    wl = synth.make_device(cfg, "cuda")
    N, B = cfg.n_keys, cfg.budget
    kb = gc.host_cache(wl["k"]).reshape(-1, N, 128)
    vb = gc.host_cache(wl["v"]).reshape(-1, N, 128)
    pb = wl["pos"].cpu().numpy().reshape(-1, N)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    rng = np.random.default_rng(44)
    raw_ids = np.sort(rng.choice(cfg.n_streams, 64, replace=False))
    _, raw = raw_scores(T, calib, wl["k"], wl["t_dev"], cfg.n_seq, N)
    raw = raw.reshape(-1, cfg.G, N)[torch.from_numpy(raw_ids).cuda()].cpu().numpy()
    F, kept = prune_all(T, calib, wl, B)
    out = {"F": F.cpu().numpy().reshape(-1, N), "kept": kept.cpu().numpy()}
    ka = gc.host_cache(wl["k"]).reshape(-1, N, 128)
    va = gc.host_cache(wl["v"]).reshape(-1, N, 128)
    pa = wl["pos"].cpu().numpy().reshape(-1, N)
    calib.free()
    host = {"cfg": cfg, "t": wl["t"], "qc": wl["qc"], "qn": wl["qn"], "rb": wl["rb"]}
    del wl
    torch.cuda.empty_cache()
    print(f"[setup] pruned {cfg.n_streams} streams on the GPU", flush=True)
    return {"cfg": cfg, "host": host, "kb": kb, "vb": vb, "pb": pb, "ka": ka, "va": va, "pa": pa, "out": out,
            "raw_ids": raw_ids, "raw": raw}


@pytest.mark.parametrize("part", range(8))
def test_config4_every_stream(orc, T, config4, part, capsys):
    """One eighth of config 4's streams per test (2304 streams, 5.0 M keys)."""
    c = config4
    cfg = c["cfg"]
    n = cfg.n_streams // 8
    ids = np.arange(part * n, (part + 1) * n)
    e_F, n_diff, _ = oracle_check_streams(orc, T, cfg, c["host"], ids, c["kb"][ids], c["vb"][ids], c["pb"][ids],
                                          c["out"], c["ka"][ids], c["va"][ids], c["pa"][ids])
    report(capsys, f"[ok] streams {ids[0]}..{ids[-1]} of {cfg.n_streams} against the oracle: F err {e_F:.2e}, "
          f"near-threshold set differences in {n_diff} streams")


def test_config4_raw_scores_sampled(orc, T, config4, capsys):
    c = config4
    cfg = c["cfg"]
    ids = c["raw_ids"]
    res = orc.prune_streams(c["kb"][ids], c["pb"][ids], c["host"]["t"], c["host"]["qc"], c["host"]["qn"],
                            c["host"]["rb"], cfg.budget, cfg.n_kv_heads, stream_ids=ids, form="fac", want_raw=True)
    e_raw = gc.check_raw(c["raw"], res["raw"])
    report(capsys, f"[ok] raw scores of {len(ids)} seeded streams: err {e_raw:.2e}")


def config5_sample(n_streams, clusters=16, rounds=256, seed=55):
    """256 streams: for each of the 16 stream clusters of the staged launch (cluster = stream mod
    16, round = stream div 16 on 256 CUs), rounds 0, 1, 2, 127, 128, 253, 254, 255 and 8 seeded
    others."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, rounds // 2 - 1, rounds // 2, rounds - 3, rounds - 2, rounds - 1]
    ids = []
    for c in range(clusters):
        others = rng.choice(np.setdiff1d(np.arange(rounds), fixed), 8, replace=False)
        ids += [r * clusters + c for r in sorted(fixed + others.tolist())]
    ids = np.array(sorted(ids))
    assert len(ids) == 256 and ids.max() < n_streams
    return ids


def test_config5_every_stream_and_oracle_sample(orc, T, capsys):
    import torch
    cfg = synth.CONFIGS[5]
    print(f"\n[case] {cfg.describe()}", flush=True)
    wl = synth.make_device(cfg, "cuda")
    N, B, G = cfg.n_keys, cfg.budget, cfg.G
    ids = config5_sample(cfg.n_streams)
    ids_t = torch.from_numpy(ids).cuda()
    k_all = wl["k"].reshape(-1, N, 128)
    kb = gc.host_cache(k_all[ids_t])
    vb = gc.host_cache(wl["v"].reshape(-1, N, 128)[ids_t])
    pb = wl["pos"].reshape(-1, N)[ids_t].cpu().numpy()
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)

    # the exchange-free tiled path and the raw-score output, on the unpruned cache
    F_tiled = T.score(calib, wl["k"], wl["t_dev"], flags=T.SCORE_TILED, check=True)
    F_raw, raw = raw_scores(T, calib, wl["k"], wl["t_dev"], cfg.n_seq, N)
    raw_s = raw.reshape(-1, G, N)[ids_t].cpu().numpy()
    del raw
    torch.cuda.empty_cache()
    # the benchmark's call on every stream
    F, kept = prune_all(T, calib, wl, B)
    assert torch.equal(F, F_raw), "final scores differ between the prune and the raw-output score calls"
    Fh = F.cpu().numpy().reshape(-1, N)
    Ft = F_tiled.cpu().numpy().reshape(-1, N).astype(np.float64)
    kh = kept.cpu().numpy()
    print("[check] every stream against the tiled path", flush=True)
    rel = np.abs(Fh.astype(np.float64) - Ft) / np.maximum(np.abs(Ft), 1.0)
    worst = float(rel.max())
    assert worst <= PATH_RTOL, f"cluster vs tiled final scores differ by {worst:.3g}"
    kt = T.select_topB(F_tiled, B).cpu().numpy()
    n_diff = 0
    for i in np.nonzero(np.any(kt != kh, axis=1))[0]:
        FB = np.sort(Ft[i])[::-1][B - 1]
        for j in np.setxor1d(kt[i], kh[i]):
            assert abs(Ft[i, j] - FB) <= PATH_RTOL * max(1.0, abs(FB)), f"stream {i}: key {j} differs off the threshold"
        n_diff += 1
    select_order_ok(Fh, kh, B)
    report(capsys, f"[ok] {cfg.n_streams} streams: cluster vs tiled F err {worst:.2e}, kept sets differ (near the threshold "
          f"only) in {n_diff} streams, selection order rule holds on every stream")

    print(f"[check] {len(ids)} streams against the oracle", flush=True)
    out = {"F": Fh, "kept": kh}
    ka = gc.host_cache(wl["k"].reshape(-1, N, 128)[ids_t])
    va = gc.host_cache(wl["v"].reshape(-1, N, 128)[ids_t])
    pa = wl["pos"].reshape(-1, N)[ids_t].cpu().numpy()
    e_F, n_diff, e_raw = oracle_check_streams(orc, T, cfg, wl, ids, kb, vb, pb, out, ka, va, pa, raw=raw_s)
    report(capsys, f"[ok] {len(ids)} of {cfg.n_streams} streams (16 clusters x first/middle/last and seeded rounds) against "
          f"the oracle: raw err {e_raw:.2e}, F err {e_F:.2e}, near-threshold set differences in {n_diff} streams")
    calib.free()
    del wl
    torch.cuda.empty_cache()
