"""GPU: the tile-parallel compaction that tria_prune takes (one block per tile of 256 destination
rows, every tile of every stream in flight), and its fallback when the workspace has no room for its
synchronisation words.

Each case compares tria_prune (score, selection, tile-parallel compaction) with the three separate
calls (score, selection, the per-stream compaction of tria_compact) on the same seeded cache, bit
for bit: F, kept indices, compacted K, V and positions, and the rows past the budget.  The kernel
timers show which compaction ran.  Rows move as chenxutan.com/d/2624 section 4.2 indexes the
cache: row i takes row kept[i], kept ascending.
"""
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


def _case(T, dtype, G, N, B, n_seq=2, n_layers=1, seed=70):
    cfg = gc.variant(2, name=f"tiles-{dtype}-N{N}-B{B}", n_q_heads=2 * G, n_kv_heads=2, n_seq=n_seq,
                     n_layers=n_layers, n_keys=N, budget=B, dtype=dtype, t_fixed=N + 300, calib="head_r",
                     r_range=(0.6, 0.99), seed=seed)
    wl = synth.make_host(cfg)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], cfg.n_kv_heads, cfg.theta)
    return cfg, wl, calib


def _separate(T, calib, d, B):
    F = T.score(calib, d["k"], d["t_dev"], check=True)
    kept = T.select_topB(F, B)
    T.compact(d["k"], d["v"], d["pos"], kept, B)
    return F, kept


def _same(torch, a, b):
    assert torch.equal(a["k"].view(torch.int16) if a["k"].dtype == torch.bfloat16 else a["k"],
                       b["k"].view(torch.int16) if b["k"].dtype == torch.bfloat16 else b["k"])
    assert torch.equal(a["v"], b["v"]) and torch.equal(a["pos"], b["pos"])


def _launches(T):
    return {name: kv["launches"] for name, kv in T.timing_read().items()}


@pytest.mark.parametrize("dtype,G,N,B,n_seq,n_layers", [
    ("bf16", 4, 3200, 3072, 1, 4),      # Qwen3-8B prune shape (128 keys evicted), few streams
    ("bf16", 4, 40000, 30000, 1, 1),    # long shifts: a tile's destinations hold sources of many earlier tiles
    ("bf16", 8, 32768, 3072, 1, 1),     # one-shot compression: most sources lie past the budget
    ("f32", 2, 3001, 1000, 2, 1),       # fp32 rows (32 words per row)
    ("bf16", 4, 5000, 257, 2, 1),       # one full tile and a one-row tile
    ("bf16", 4, 600, 200, 2, 1),        # one partial tile
    ("bf16", 4, 1025, 1024, 2, 1),      # one key evicted
    ("bf16", 4, 700, 1, 2, 1),          # budget 1
])
def test_tile_compaction_matches_per_stream_compaction(T, dtype, G, N, B, n_seq, n_layers):
    import torch
    print(f"\n[case] tile compaction {dtype} G={G} N={N} B={B} streams={n_seq * n_layers * 2}", flush=True)
    cfg, wl, calib = _case(T, dtype, G, N, B, n_seq=n_seq, n_layers=n_layers)
    d1, d2 = synth.to_device(wl), synth.to_device(wl)
    k0 = d2["k"].clone()
    F1, kept1 = _separate(T, calib, d1, B)
    torch.cuda.synchronize()
    T.timing_enable(True)
    try:
        T.timing_read()
        F2, kept2 = T.prune(calib, d2["k"], d2["v"], d2["pos"], d2["t_dev"], B)
        torch.cuda.synchronize()
        n = _launches(T)
    finally:
        T.timing_enable(False)
    assert n["compact"] == 1 and n["select"] == 1 and n["select_compact"] == 0, n
    assert torch.equal(F1, F2) and torch.equal(kept1, kept2)
    _same(torch, d1, d2)
    # rows past the budget are left as they were
    assert torch.equal(d2["k"][..., B:, :], k0[..., B:, :])
    calib.free()


def test_tile_compaction_ignores_workspace_contents(T):
    """The selection clears the compaction's counter and flags on every call: a workspace filled
    with 0xff bytes, and two calls in a row on the same workspace, give the same results."""
    import torch
    print("\n[case] tile compaction, workspace of 0xff bytes, two calls", flush=True)
    cfg, wl, calib = _case(T, "bf16", 4, 3200, 3072, n_seq=1, n_layers=3, seed=71)
    ref = synth.to_device(wl)
    F1, kept1 = _separate(T, calib, ref, cfg.budget)
    S, N = cfg.n_seq, cfg.n_keys
    ws = T.workspace(T.prune_workspace_bytes(calib, S, N, cfg.budget))
    assert ws.numel() > T.score_workspace_bytes(calib, S, N)
    for call in range(2):
        d = synth.to_device(wl)
        ws.fill_(0xff)
        torch.cuda.synchronize()
        F2, kept2 = T.prune(calib, d["k"], d["v"], d["pos"], d["t_dev"], cfg.budget, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(F1, F2) and torch.equal(kept1, kept2), f"call {call}"
        _same(torch, ref, d)
    calib.free()


def test_score_sized_workspace_takes_the_per_stream_compaction(T):
    """A workspace with room for the score only: tria_prune falls back to the fused per-stream
    selection and compaction, with the same results."""
    import torch
    print("\n[case] tile compaction fallback, score-sized workspace", flush=True)
    cfg, wl, calib = _case(T, "bf16", 4, 3200, 3072, n_seq=1, n_layers=2, seed=72)
    ref = synth.to_device(wl)
    F1, kept1 = _separate(T, calib, ref, cfg.budget)
    d = synth.to_device(wl)
    ws = T.workspace(T.score_workspace_bytes(calib, cfg.n_seq, cfg.n_keys))
    torch.cuda.synchronize()
    T.timing_enable(True)
    try:
        T.timing_read()
        F2, kept2 = T.prune(calib, d["k"], d["v"], d["pos"], d["t_dev"], cfg.budget, ws=ws)
        torch.cuda.synchronize()
        n = _launches(T)
    finally:
        T.timing_enable(False)
    assert n["select_compact"] == 1 and n["compact"] == 0, n
    assert torch.equal(F1, F2) and torch.equal(kept1, kept2)
    _same(torch, ref, d)
    calib.free()


@pytest.mark.parametrize("word,status", [(0, "OK"), (1, "E_NONFINITE"), (2, "E_DEVICE"), (4, "E_DEVICE"),
                                         (5, "E_DEVICE")])
def test_score_check_reads_every_error_bit(T, word, status):
    """The step's error word (the workspace's first int): bit 0 a non-finite score, bit 1 a stream
    cluster's exchange that did not complete, bit 2 a tile of the tile-parallel compaction whose
    wait ran past its bound.  tria_score_check reports the first as TRIA_E_NONFINITE and the
    others as TRIA_E_DEVICE (set here from the host; no kernel is made to fail)."""
    import torch
    ws = T.workspace(256)
    ws.zero_()
    ws[:4].copy_(torch.tensor([word], dtype=torch.int32).view(torch.uint8))
    torch.cuda.synchronize()
    if status == "OK":
        T.score_check(ws)
        return
    with pytest.raises(T.TriaError) as e:
        T.score_check(ws)
    assert e.value.status == getattr(T, status)


def test_tile_compaction_without_positions(T):
    """No positions array (pos = NULL): K and V move as with the per-stream compaction."""
    import torch
    print("\n[case] tile compaction without positions", flush=True)
    cfg, wl, calib = _case(T, "bf16", 4, 3200, 3072, n_seq=1, n_layers=2, seed=73)
    d1, d2 = synth.to_device(wl), synth.to_device(wl)
    F1 = T.score(calib, d1["k"], d1["t_dev"], check=True)
    kept1 = T.select_topB(F1, cfg.budget)
    T.compact(d1["k"], d1["v"], None, kept1, cfg.budget)
    F2, kept2 = T.prune(calib, d2["k"], d2["v"], None, d2["t_dev"], cfg.budget)
    torch.cuda.synchronize()
    assert torch.equal(F1, F2) and torch.equal(kept1, kept2)
    assert torch.equal(d1["k"].view(torch.int16), d2["k"].view(torch.int16))
    assert torch.equal(d1["v"].view(torch.int16), d2["v"].view(torch.int16))
    calib.free()
