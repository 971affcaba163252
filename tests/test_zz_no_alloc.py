"""The allocation-free prune step (tria_prune_static, scratch in the library's static device array)
against tria_prune with a caller workspace, through the C ABI, on two calls in a row: first the
Qwen3-8B batch-64 cache (18432 streams of 2176 keys: its workspace does not fit the array, so the
call runs in chunks of whole sequences), then a smaller Qwen3-32B-shaped cache (16 streams of
32768 keys, the stream-cluster path).  F, kept indices and the compacted K, V and positions must be
the same bits; the device's free memory must not change during a call."""
import dataclasses

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
    # set-up: the first call on a device looks up the array (the runtime has placed it with the
    # library's code) and the first launches of each path load their kernels; later calls allocate
    # nothing
    for base, name in ((4, "warm-c4"), (5, "warm-c5")):
        cfg = dataclasses.replace(synth.CONFIGS[base], name=name, n_seq=1, n_layers=1)
        wl = synth.make_device(cfg, "cuda")
        calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
        T.prune_static(calib, wl["k"], wl["v"], wl["pos"], wl["t_dev"], cfg.budget)
        calib.free()
        del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return T


def compare_with_prune(T, cfg):
    import torch
    print(f"\n[case] static-workspace prune vs tria_prune: {cfg.describe()}", flush=True)
    wl = synth.make_device(cfg, "cuda")
    k1, v1, p1 = wl["k"], wl["v"], wl["pos"]
    k2, v2, p2 = k1.clone(), v1.clone(), p1.clone()
    S, L, Hkv, N, _ = k1.shape
    B = cfg.budget
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    F1, kept1 = T.prune(calib, k1, v1, p1, wl["t_dev"], B)
    # outputs of the static call are allocated here, before the call: the call itself allocates nothing
    F2 = torch.empty_like(F1)
    kept2 = torch.empty_like(kept1)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    _, _, addr = T.prune_static(calib, k2, v2, p2, wl["t_dev"], B, F=F2, kept=kept2)   # waits, checks
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    chunk_ws = T.prune_workspace_bytes(calib, S, N, B)
    print(f"[info] caller workspace {chunk_ws / 2**20:.1f} MiB for all {S} sequences; static array "
          f"{T.STATIC_WORKSPACE_BYTES / 2**20:.0f} MiB at {addr:#x}; free device memory {free0} -> {free1}", flush=True)
    assert free1 == free0, "device memory was allocated during the call"
    assert torch.equal(F1.view(torch.int32), F2.view(torch.int32)), "final scores differ"
    assert torch.equal(kept1, kept2), "kept indices differ"
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16)) and torch.equal(v1.view(torch.int16), v2.view(torch.int16))
    assert torch.equal(p1, p2)
    calib.free()
    del wl, k2, v2, p2
    torch.cuda.empty_cache()
    return chunk_ws


def test_static_workspace_two_calls(T):
    big = synth.CONFIGS[4]
    small = dataclasses.replace(synth.CONFIGS[5], name="qwen3-32b-shape-1seq-2layer", n_seq=1, n_layers=2)
    ws_big = compare_with_prune(T, big)
    assert ws_big > T.STATIC_WORKSPACE_BYTES, "the first call should need several chunks"
    compare_with_prune(T, small)


def test_static_workspace_rejects_what_does_not_fit(T):
    """One sequence whose workspace exceeds the array (the tiled path stages raw scores of every
    head in HBM): a clear TRIA_E_WORKSPACE, and nothing runs."""
    import torch
    cfg = dataclasses.replace(synth.CONFIGS[5], name="qwen3-32b-shape-tiled", n_seq=1)   # 537 MB of raw scores
    wl = synth.make_device(cfg, "cuda")
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    k0 = wl["k"].clone()
    F = torch.zeros((1, cfg.n_layers, cfg.n_kv_heads, cfg.n_keys), dtype=torch.float32, device="cuda")
    with pytest.raises(T.TriaError) as e:
        T.prune_static(calib, wl["k"], wl["v"], wl["pos"], wl["t_dev"], cfg.budget, F=F, flags=T.SCORE_TILED)
    assert e.value.status == T.E_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(wl["k"].view(torch.int16), k0.view(torch.int16))
    calib.free()
