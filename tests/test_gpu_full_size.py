"""GPU parity at the full sizes of the large workloads, in the launch configuration the benchmark
times: every stream is scored, selected and compacted on the GPU; the oracle recomputes a seeded
sample of streams (scores, selection, compaction of K, V and positions)."""
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


@pytest.mark.parametrize("cfg_id,n_sample", [(4, 12), (5, 6)])
def test_full_size_sampled_streams(orc, T, cfg_id, n_sample):
    import torch
    cfg = synth.CONFIGS[cfg_id]
    print(f"\n[case] full size {cfg.describe()}", flush=True)
    wl = synth.make_device(cfg, "cuda")
    N, B = cfg.n_keys, cfg.budget
    rng = np.random.default_rng(1000 + cfg_id)
    ids = np.sort(rng.choice(cfg.n_streams, n_sample, replace=False))
    ids_t = torch.from_numpy(ids).cuda()
    kb = gc.host_cache(wl["k"].reshape(-1, N, 128)[ids_t])
    vb = gc.host_cache(wl["v"].reshape(-1, N, 128)[ids_t])
    pb = wl["pos"].reshape(-1, N)[ids_t].cpu().numpy()
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    out = gc.gpu_prune(T, calib, wl, B, want_raw=False)
    res = orc.prune_streams(kb, pb, wl["t"], wl["qc"], wl["qn"], wl["rb"], B, cfg.n_kv_heads, stream_ids=ids,
                            form="fac")
    e_F = gc.check_F(out["F"][ids], res["F"])
    n_diff = gc.check_kept_sets(out["kept"][ids], res["kept"], res["F"], B)
    gc.check_select_exact(orc, out["kept"][ids], out["F"][ids], B)
    ka = gc.host_cache(wl["k"].reshape(-1, N, 128)[ids_t])
    va = gc.host_cache(wl["v"].reshape(-1, N, 128)[ids_t])
    pa = wl["pos"].reshape(-1, N)[ids_t].cpu().numpy()
    gc.check_compaction(kb, ka, out["kept"][ids], B)
    gc.check_compaction(vb, va, out["kept"][ids], B)
    gc.check_compaction(pb, pa, out["kept"][ids], B)
    # every stream: kept strictly ascending, in range, B of them
    kept = out["kept"]
    assert kept.shape == (cfg.n_streams, min(B, N))
    assert np.all(np.diff(kept, axis=1) > 0) and kept.min() >= 0 and kept.max() < N
    print(f"[ok] F err {e_F:.2e}, streams with near-threshold differences {n_diff}", flush=True)
    calib.free()
    del wl
    torch.cuda.empty_cache()
