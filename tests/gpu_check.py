"""Helpers of the GPU parity tests: run the HIP path through the C ABI and compare it with the
fp64 oracle on the same seeded inputs.

Tolerances (fp32 accumulation against fp64):
  raw scores   |s_gpu - s_orc| <= 1e-4 * max(|s_orc|, std_h)      (std_h: the head's oracle std)
  final score  |F_gpu - F_orc| <= 1e-4 * max(|F_orc|, 1)
  kept sets    identical except keys whose oracle score lies within 1e-4 * max(1, |F_B|) of the
               oracle's B-th largest score F_B
  selection    bit-exact against the oracle's selection run on the GPU's own final scores
  compaction   bit-exact against fancy indexing of a pristine copy
"""
from __future__ import annotations

import dataclasses

import numpy as np

import synth

RAW_RTOL = 1e-4
F_RTOL = 1e-4


def gpu_prune(T, calib, dev, budget, want_raw=True, flags=0):
    """Score, select and compact through the C ABI; returns host copies of everything."""
    import torch

    k, v, pos, t = dev["k"], dev["v"], dev["pos"], dev["t_dev"]
    S, L, Hkv, N, d = k.shape
    Hq = calib.n_q_heads
    raw = torch.empty((S, L, Hq, N), dtype=torch.float32, device=k.device) if want_raw else None
    stats = torch.empty((S, L, Hq, 2), dtype=torch.float32, device=k.device)
    ws = T.workspace(T.score_workspace_bytes(calib, S, N, k.dtype, flags), k.device)
    F = T.score(calib, k, t, raw=raw, head_stats=stats, pos=pos, flags=flags, ws=ws)
    T.score_check(ws)
    kept = T.select_topB(F, budget)
    T.compact(k, v, pos, kept, budget)
    torch.cuda.synchronize()
    out = {"F": F.cpu().numpy().reshape(-1, N), "kept": kept.cpu().numpy(),
           "stats": stats.cpu().numpy().reshape(-1, calib.G, 2)}
    if want_raw:
        out["raw"] = raw.cpu().numpy().reshape(-1, calib.G, N)
    return out


def oracle_prune(orc, wl_host_streams, pos_streams, t, qc, qn, rb, budget, Hkv, ids, form):
    return orc.prune_streams(wl_host_streams, pos_streams, t, qc, qn, rb, budget, Hkv, stream_ids=ids,
                             form=form, want_raw=True)


def check_raw(raw_gpu, raw_orc):
    """raw_* [n][G][N]."""
    sd = raw_orc.std(axis=2, keepdims=True)
    scale = np.maximum(np.abs(raw_orc), sd)
    err = np.abs(raw_gpu.astype(np.float64) - raw_orc) / scale
    assert np.all(np.isfinite(raw_gpu))
    worst = float(err.max())
    assert worst <= RAW_RTOL, f"raw score relative error {worst:.3g} > {RAW_RTOL}"
    return worst


def check_F(F_gpu, F_orc):
    err = np.abs(F_gpu.astype(np.float64) - F_orc) / np.maximum(np.abs(F_orc), 1.0)
    worst = float(err.max())
    assert worst <= F_RTOL, f"final score relative error {worst:.3g} > {F_RTOL}"
    return worst


def check_kept_sets(kept_gpu, kept_orc, F_orc, budget):
    """Sets may differ only on near-threshold keys (by the oracle's scores).  Both lists are
    ascending, so equal sets are equal rows."""
    n, N = F_orc.shape
    n_diff = 0
    for i in np.nonzero(np.any(np.asarray(kept_gpu) != np.asarray(kept_orc), axis=1))[0]:
        a, b = set(kept_gpu[i].tolist()), set(kept_orc[i].tolist())
        if a == b:
            continue
        nk = min(budget, N)
        FB = np.sort(F_orc[i])[::-1][nk - 1]
        tol = 1e-4 * max(1.0, abs(FB))
        for j in a ^ b:
            assert abs(F_orc[i, j] - FB) <= tol, f"stream {i}: key {j} differs and is not near the threshold"
        n_diff += 1
    return n_diff


def check_select_exact(orc, kept_gpu, F_gpu, budget):
    for i in range(F_gpu.shape[0]):
        ref = orc.select(F_gpu[i].astype(np.float64), budget)
        assert np.array_equal(kept_gpu[i], ref), f"stream {i}: selection differs from a full sort"


def check_compaction(before, after, kept, budget, chunk=512):
    """before/after [n][N][...] host arrays of one tensor; kept [n][nk].  Rows [0, nk) of every
    stream must equal its rows kept[i] of the pristine copy (fancy indexing), bit for bit, and
    rows past nk must be untouched."""
    n, N = before.shape[0], before.shape[1]
    nk = min(budget, N)
    kept = np.asarray(kept)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        idx = kept[c0:c1].reshape(kept[c0:c1].shape + (1,) * (before.ndim - 2))
        exp = np.take_along_axis(before[c0:c1], idx, axis=1)
        bad = np.nonzero(np.any((after[c0:c1, :nk] != exp).reshape(c1 - c0, -1), axis=1))[0]
        assert bad.size == 0, f"stream {c0 + bad[0]}: compacted rows differ"
        bad = np.nonzero(np.any((after[c0:c1, nk:] != before[c0:c1, nk:]).reshape(c1 - c0, -1), axis=1))[0]
        assert bad.size == 0, f"stream {c0 + bad[0]}: rows past B were touched"


def streams_of(x, N):
    """[S][L][Hkv][N][...] -> [streams][N][...]"""
    return x.reshape((-1, N) + x.shape[4:])


def host_cache(x):
    return synth.cache_to_host(x)


def variant(base: int, **kw):
    return dataclasses.replace(synth.CONFIGS[base], **kw)


def run_case(orc, T, cfg, form="fac", sample=None, flags=0):
    print(f"\n[case] {cfg.describe()} form={form} flags={flags}", flush=True)
    pre_rope = bool(flags & T.KEYS_PRE_ROPE)
    weight_r = bool(flags & T.TRIG_WEIGHT_R)
    wl = synth.make_host(cfg, pre_rope=pre_rope)
    dev = synth.to_device(wl)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    N, B = cfg.n_keys, cfg.budget
    kb, vb, pb = streams_of(wl["k"], N), streams_of(wl["v"], N), streams_of(wl["pos"], N)
    out = gpu_prune(T, calib, dev, B, flags=flags)
    ids = np.arange(cfg.n_streams) if sample is None else np.asarray(sample)
    res = orc.prune_streams(kb[ids], pb[ids], wl["t"], wl["qc"], wl["qn"], wl["rb"], B, cfg.n_kv_heads,
                            stream_ids=ids, form=form, want_raw=True, pre_rope=pre_rope, weight_r=weight_r)
    e_raw = check_raw(out["raw"][ids], res["raw"])
    e_F = check_F(out["F"][ids], res["F"])
    n_diff = check_kept_sets(out["kept"][ids], res["kept"], res["F"], B)
    check_select_exact(orc, out["kept"][ids], out["F"][ids], B)
    mu = res["raw"].mean(axis=2)
    sd = res["raw"].std(axis=2)
    np.testing.assert_allclose(out["stats"][ids, :, 0], mu, rtol=1e-5, atol=1e-5 * np.abs(sd).max())
    np.testing.assert_allclose(out["stats"][ids, :, 1], sd, rtol=1e-4)
    ka = streams_of(host_cache(dev["k"]), N)
    va = streams_of(host_cache(dev["v"]), N)
    pa = streams_of(dev["pos"].cpu().numpy(), N)
    check_compaction(kb[ids], ka[ids], out["kept"][ids], B)
    check_compaction(vb[ids], va[ids], out["kept"][ids], B)
    check_compaction(pb[ids], pa[ids], out["kept"][ids], B)
    print(f"[ok] raw err {e_raw:.2e}  F err {e_F:.2e}  streams with near-threshold set differences {n_diff}",
          flush=True)
    calib.free()
    return out, res
