"""GPU tests of the decode loop: appending generated rows (tria_append) and the append-then-prune
step (tria_decode_step) against the fp64 oracle run the same way.

The loop keeps a cache of capacity B + 128 per stream: each round appends the K/V rows of 128
new tokens (positions t+1 .. t+128, post-RoPE keys drawn with the synthetic recipe) and, the
cache being full, prunes it back to B.  In lockstep, every round's pre-prune cache (the GPU's
own) is pruned by the oracle; kept sets must agree up to near-threshold keys and the compacted
cache must equal the oracle's compaction of that same cache bit for bit.  A second, independent
oracle run of all rounds from the same start must end on the same positions when no round had a
near-threshold difference.
"""
import math

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


def new_rows(rng, centres, pos, dtype):
    """Post-RoPE K rows of new tokens and V rows: centres [L][Hkv][d]; pos [S][L][Hkv][n]."""
    S, L, Hkv, n = pos.shape
    w = synth.omega_table()
    pre = centres[None, :, :, None, :] + 0.5 * rng.standard_normal((S, L, Hkv, n, 128))
    k = synth.rope_fp64(pre, pos, w).astype(np.float32)
    v = rng.standard_normal((S, L, Hkv, n, 128)).astype(np.float32)
    if dtype == "bf16":
        return synth.f32_to_bf16_bits(k), synth.f32_to_bf16_bits(v)
    return k, v


def dev_cache(x, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_copies_rows(T, dtype):
    import torch
    print(f"\n[case] append {dtype}", flush=True)
    rng = np.random.default_rng(600)
    S, L, Hkv, cap, n, length = 2, 3, 2, 200, 37, 101
    kc = rng.standard_normal((S, L, Hkv, cap, 128)).astype(np.float32)
    vc = rng.standard_normal((S, L, Hkv, cap, 128)).astype(np.float32)
    pc = rng.integers(0, 10000, (S, L, Hkv, cap)).astype(np.int32)
    kn = rng.standard_normal((S, L, Hkv, n, 128)).astype(np.float32)
    vn = rng.standard_normal((S, L, Hkv, n, 128)).astype(np.float32)
    pn = rng.integers(0, 10000, (S, L, Hkv, n)).astype(np.int32)
    if dtype == "bf16":
        kc, vc, kn, vn = (synth.f32_to_bf16_bits(x) for x in (kc, vc, kn, vn))
    dk, dv, dn_k, dn_v = (dev_cache(x, dtype) for x in (kc, vc, kn, vn))
    dp, dn_p = torch.from_numpy(pc).cuda(), torch.from_numpy(pn).cuda()
    T.append(dk, dv, dp, length, dn_k, dn_v, dn_p)
    torch.cuda.synchronize()
    ek, ev, ep = kc.copy(), vc.copy(), pc.copy()
    ek[:, :, :, length:length + n] = kn
    ev[:, :, :, length:length + n] = vn
    ep[:, :, :, length:length + n] = pn
    assert np.array_equal(synth.cache_to_host(dk), ek)
    assert np.array_equal(synth.cache_to_host(dv), ev)
    assert np.array_equal(dp.cpu().numpy(), ep)
    with pytest.raises(T.TriaError):
        T.append(dk, dv, dp, cap - n + 1, dn_k, dn_v, dn_p)      # would run past the capacity


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f32", 2), ("bf16", 8)])
def test_decode_loop_matches_oracle(T, orc, dtype, G):
    import torch
    print(f"\n[case] decode loop {dtype} G={G}", flush=True)
    rng = np.random.default_rng(610 + G)
    S, L, Hkv, B, rounds = 2, 2, 2, 256, 5
    cap = B + 128
    cfg = gc.variant(2, name="decode", n_layers=L, n_seq=S, n_q_heads=Hkv * G, n_kv_heads=Hkv, n_keys=B,
                     budget=B, dtype=dtype, t_fixed=3000, calib="head_r", r_range=(0.6, 0.99), seed=620 + G)
    wl = synth.make_host(cfg)                       # the prefill: B rows per stream at gapped positions
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], Hkv, cfg.theta)
    u = rng.standard_normal((L, Hkv, 128))
    centres = 8.0 * u / np.linalg.norm(u, axis=-1, keepdims=True)
    kdt = np.uint16 if dtype == "bf16" else np.float32
    hk = np.zeros((S, L, Hkv, cap, 128), kdt)
    hv = np.zeros((S, L, Hkv, cap, 128), kdt)
    hp = np.zeros((S, L, Hkv, cap), np.int32)
    hk[:, :, :, :B], hv[:, :, :, :B], hp[:, :, :, :B] = wl["k"], wl["v"], wl["pos"]
    dk, dv = dev_cache(hk, dtype), dev_cache(hv, dtype)
    dp = torch.from_numpy(hp).cuda()
    # independent oracle state (host), from the same start
    ok, ov, op = hk.copy(), hv.copy(), hp.copy()
    t = np.full(S, 3000, np.int32)
    n_near = 0
    streams = S * L * Hkv
    length = B
    for r in range(rounds):
        pos_new = (t[:, None, None, None] + 1 + np.arange(128, dtype=np.int32)).astype(np.int32)
        pos_new = np.broadcast_to(pos_new, (S, L, Hkv, 128)).copy()
        kn, vn = new_rows(rng, centres, pos_new, dtype)
        t = t + 128
        before_k = synth.cache_to_host(dk).copy()
        before_v = synth.cache_to_host(dv).copy()
        before_p = dp.cpu().numpy().copy()
        kept = torch.empty((streams, B), dtype=torch.int32, device="cuda")
        new_len = T.decode_step(calib, dk, dv, dp, torch.from_numpy(t).cuda(), length, B, dev_cache(kn, dtype),
                                dev_cache(vn, dtype), torch.from_numpy(pos_new).cuda(), kept=kept)
        torch.cuda.synchronize()
        assert new_len == B
        # lockstep: the oracle prunes the GPU's own pre-prune cache
        full_k, full_v, full_p = before_k, before_v, before_p
        full_k[:, :, :, length:] = kn
        full_v[:, :, :, length:] = vn
        full_p[:, :, :, length:] = pos_new
        res = orc.prune_streams(gc.streams_of(full_k, cap), gc.streams_of(full_p, cap), t, wl["qc"], wl["qn"],
                                wl["rb"], B, Hkv, form="fac")
        g_kept = kept.cpu().numpy()
        n_near += gc.check_kept_sets(g_kept, res["kept"], res["F"], B)
        gk = gc.streams_of(synth.cache_to_host(dk), cap)
        gv = gc.streams_of(synth.cache_to_host(dv), cap)
        gp = gc.streams_of(dp.cpu().numpy(), cap)
        gc.check_compaction(gc.streams_of(full_k, cap), gk, g_kept, B)
        gc.check_compaction(gc.streams_of(full_v, cap), gv, g_kept, B)
        gc.check_compaction(gc.streams_of(full_p, cap), gp, g_kept, B)
        # independent oracle run
        ok[:, :, :, B:], ov[:, :, :, B:], op[:, :, :, B:] = kn, vn, pos_new
        res2 = orc.prune_streams(gc.streams_of(ok, cap), gc.streams_of(op, cap), t, wl["qc"], wl["qn"], wl["rb"], B,
                                 Hkv, form="fac")
        for i in range(streams):
            s, rest = divmod(i, L * Hkv)
            l, g = divmod(rest, Hkv)
            sel = res2["kept"][i]
            ok[s, l, g, :B] = ok[s, l, g, sel]
            ov[s, l, g, :B] = ov[s, l, g, sel]
            op[s, l, g, :B] = op[s, l, g, sel]
        length = B
        print(f"[ok] round {r}: t = {t.tolist()}, streams with near-threshold set differences so far {n_near}",
              flush=True)
    if n_near == 0:
        assert np.array_equal(dp.cpu().numpy()[:, :, :, :B], op[:, :, :, :B])
    calib.free()


def test_decode_step_appends_without_pruning_until_full(T):
    """Below capacity the step only appends: no prune, the live length grows by n_new."""
    import torch
    print("\n[case] decode partial", flush=True)
    cfg = gc.variant(2, name="decode-partial", n_layers=1, n_seq=1, n_q_heads=4, n_kv_heads=1, n_keys=200,
                     budget=200, t_fixed=1000, seed=630)
    wl = synth.make_host(cfg)
    calib = T.load_calib(wl["qc"], wl["qn"], wl["rb"], 1, cfg.theta)
    cap = 456
    k = torch.zeros((1, 1, 1, cap, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    p = torch.zeros((1, 1, 1, cap), dtype=torch.int32, device="cuda")
    kn = torch.ones((1, 1, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    pn = torch.arange(128, dtype=torch.int32, device="cuda").view(1, 1, 1, 128)
    t = torch.tensor([1127], dtype=torch.int32, device="cuda")
    n = T.decode_step(calib, k, v, p, t, 200, 328, kn, kn, pn)
    torch.cuda.synchronize()
    assert n == 328
    assert torch.equal(p[0, 0, 0, 200:328].cpu(), pn.view(-1).cpu())
    calib.free()
