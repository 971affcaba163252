"""Seeded synthetic workloads for the TriAttention prune step.

This module only draws inputs: KV caches, key positions, current positions and the calibration
statistics a model would have produced offline.  It holds none of the prune step's own
arithmetic (no scoring, normalisation, selection or compaction), and both the HIP library's
tests and the oracle read their inputs from here.

Recipe (the pages measure on Qwen3-8B / Qwen3-32B with real reasoning traces; no weights or
datasets are available, so these synthetic caches stand in for them):
  * head_dim d = 128, half-split RoPE (band f pairs dims f and f+64), theta = 1e6,
    w_f = fl32(theta^(-2f/d)).
  * Per (layer, KV head) a key centre c = 8*u/|u|, u ~ N(0, I_d); a pre-RoPE key is c + n with
    n ~ N(0, 0.5^2) per dim (the pre-RoPE concentration the pages describe).  The key is rotated
    to its position p in fp64, then rounded to the cache dtype (fp32, or bf16 with
    round-to-nearest-even).  V ~ N(0, 1) in the cache dtype.
  * Per (layer, query head) a query centre qbar = 8*u/|u|.
  * Calibration statistics, one of:
      "uniform_r"  R_f ~ U(lo, hi) per band, E|q_f| = |qbar_f| / R_f;
      "queries"    4096 synthetic pre-RoPE queries qbar + N(0, 0.5^2); the centre is their mean,
                   E|q_f| the mean band norm and R_f = |E q_f| / E|q_f|, all in fp64;
      "head_r"     one R per (layer, query head) ~ U(lo, hi), broadcast to every band,
                   E|q_f| = |qbar_f| / R.
  * Positions: the 128 newest keys sit at t-127 .. t; the older survivors are sorted distinct
    uniform draws from [0, t-128], one draw per stream; or contiguous 0..N-1.

Configurations (sizes of the workloads the library is exercised on):
  1  1 layer, 1 seq, 4 q / 1 kv heads, N = 1152, B = 1024, fp32,  t = 4000, uniform_r(0.85, 0.99)
  2  1 layer, 1 seq, 32 q / 8 kv,      N = 2176, B = 2048, bf16,  t = 16383, queries
  3  36 layers, 1 seq, 32 q / 8 kv,    N = 3200, B = 3072, bf16,  t = 32767, queries per layer
  4  36 layers, 64 seqs, 32 q / 8 kv,  N = 2176, B = 2048, bf16,  t_s ~ U{4096..24575}, queries
  5  64 layers, 8 seqs, 64 q / 8 kv,   N = 32768, B = 3072, bf16, positions 0..32767,
     head_r(0.6, 0.99)
Configurations 1-3 are drawn with numpy (PCG64) on the host and reproduce bit for bit anywhere;
4-5 are drawn with torch directly in device memory (the parity checks read the device bits).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HEAD_DIM = 128
THETA = 1e6
OFFSETS = tuple(2 ** i for i in range(17))


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    n_layers: int
    n_seq: int
    n_q_heads: int
    n_kv_heads: int
    n_keys: int
    budget: int
    dtype: str            # "f32" or "bf16"
    positions: str        # "gapped" or "contiguous"
    t_fixed: int | None   # t for every sequence, or None for per-sequence draws
    t_range: tuple | None
    calib: str            # "uniform_r", "queries", "head_r"
    r_range: tuple
    seed: int
    head_dim: int = HEAD_DIM
    theta: float = THETA

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_streams(self) -> int:
        return self.n_seq * self.n_layers * self.n_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def describe(self) -> str:
        return (f"{self.name}: L={self.n_layers} S={self.n_seq} Hq={self.n_q_heads} "
                f"Hkv={self.n_kv_heads} N={self.n_keys} B={self.budget} {self.dtype}")


CONFIGS = {
    1: Config("tiny-1layer-4q1kv-N1152-fp32", 1, 1, 4, 1, 1152, 1024, "f32", "gapped", 4000, None,
              "uniform_r", (0.85, 0.99), 1),
    2: Config("qwen3-8b-1layer-N2176-bf16", 1, 1, 32, 8, 2176, 2048, "bf16", "gapped", 16383, None,
              "queries", (0.0, 0.0), 2),
    3: Config("qwen3-8b-36layer-N3200-bf16", 36, 1, 32, 8, 3200, 3072, "bf16", "gapped", 32767, None,
              "queries", (0.0, 0.0), 3),
    4: Config("qwen3-8b-36layer-batch64-N2176-bf16", 36, 64, 32, 8, 2176, 2048, "bf16", "gapped", None,
              (4096, 24575), "queries", (0.0, 0.0), 4),
    5: Config("qwen3-32b-64layer-batch8-N32768-bf16", 64, 8, 64, 8, 32768, 3072, "bf16", "contiguous",
              32767, None, "head_r", (0.6, 0.99), 5),
}


def omega_table(d: int = HEAD_DIM, theta: float = THETA) -> np.ndarray:
    """w_f = fl32(theta^(-2f/d)), f < d/2, as float64 holding the fp32 values."""
    f = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * f / d).astype(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _unit(rng, shape, d):
    u = rng.standard_normal(shape + (d,))
    return u / np.linalg.norm(u, axis=-1, keepdims=True)


def rope_fp64(x: np.ndarray, pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Rotate half-split vectors x [..., N, d] to positions pos [..., N] in fp64."""
    h = x.shape[-1] // 2
    a = pos.astype(np.float64)[..., None] * w  # exact: fp32 w times an integer below 2^31
    c, s = np.cos(a), np.sin(a)
    xr, xi = x[..., :h], x[..., h:]
    return np.concatenate([xr * c - xi * s, xr * s + xi * c], axis=-1)


def draw_positions(rng, n_keys: int, t: int, mode: str, recent: int = 128) -> np.ndarray:
    if mode == "contiguous":
        return np.arange(t - n_keys + 1, t + 1, dtype=np.int32)
    n_old = n_keys - recent
    old = np.sort(rng.choice(t - recent + 1, size=n_old, replace=False)).astype(np.int32)
    new = np.arange(t - recent + 1, t + 1, dtype=np.int32)
    return np.concatenate([old, new])


def draw_calibration(rng, cfg: Config, L: int | None = None):
    """Returns (qc [L][Hq][d], qn [L][Hq][d/2], rb [L][Hq][d/2]) as float32."""
    L = cfg.n_layers if L is None else L
    d, h, Hq = cfg.head_dim, cfg.head_dim // 2, cfg.n_q_heads
    qbar = 8.0 * _unit(rng, (L, Hq), d)
    if cfg.calib == "uniform_r":
        R = rng.uniform(cfg.r_range[0], cfg.r_range[1], size=(L, Hq, h))
        qc = qbar
        mag = np.hypot(qc[..., :h], qc[..., h:])
        E = mag / R
    elif cfg.calib == "head_r":
        R = np.broadcast_to(rng.uniform(cfg.r_range[0], cfg.r_range[1], size=(L, Hq, 1)), (L, Hq, h))
        qc = qbar
        mag = np.hypot(qc[..., :h], qc[..., h:])
        E = mag / R
    elif cfg.calib == "queries":
        n_cal = 4096
        qc = np.empty((L, Hq, d))
        E = np.empty((L, Hq, h))
        R = np.empty((L, Hq, h))
        for l in range(L):
            q = qbar[l][:, None, :] + 0.5 * rng.standard_normal((Hq, n_cal, d))
            m = q.mean(axis=1)
            bn = np.hypot(q[..., :h], q[..., h:]).mean(axis=1)
            qc[l] = m
            E[l] = bn
            R[l] = np.hypot(m[:, :h], m[:, h:]) / bn
    else:
        raise ValueError(cfg.calib)
    return (np.ascontiguousarray(qc, dtype=np.float32), np.ascontiguousarray(E, dtype=np.float32),
            np.ascontiguousarray(R, dtype=np.float32))


def make_host(cfg: Config, n_seq: int | None = None, n_layers: int | None = None, pre_rope: bool = False):
    """Draw a whole workload on the host with numpy.

    Returns a dict: k, v [S][L][Hkv][N][d] (float32 or uint16 bf16 bits), pos [S][L][Hkv][N]
    int32, t [S] int32, qc [L][Hq][d], qn, rb [L][Hq][d/2] float32, plus the config.
    With ``pre_rope`` the cache holds the keys before RoPE (same draws, no rotation).
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    S = cfg.n_seq if n_seq is None else n_seq
    L = cfg.n_layers if n_layers is None else n_layers
    Hkv, N, d = cfg.n_kv_heads, cfg.n_keys, cfg.head_dim
    w = omega_table(d, cfg.theta)
    qc, qn, rb = draw_calibration(rng, cfg, L)
    if cfg.t_fixed is not None:
        t = np.full(S, cfg.t_fixed, dtype=np.int32)
    else:
        t = rng.integers(cfg.t_range[0], cfg.t_range[1] + 1, size=S).astype(np.int32)
    kc = 8.0 * _unit(rng, (L, Hkv), d)
    kdt = np.float32 if cfg.dtype == "f32" else np.uint16
    k = np.empty((S, L, Hkv, N, d), dtype=kdt)
    v = np.empty((S, L, Hkv, N, d), dtype=kdt)
    pos = np.empty((S, L, Hkv, N), dtype=np.int32)
    for s in range(S):
        for l in range(L):
            for g in range(Hkv):
                pos[s, l, g] = draw_positions(rng, N, int(t[s]), cfg.positions)
            pre = kc[l][:, None, :] + 0.5 * rng.standard_normal((Hkv, N, d))
            post = (pre if pre_rope else rope_fp64(pre, pos[s, l], w)).astype(np.float32)
            vv = rng.standard_normal((Hkv, N, d)).astype(np.float32)
            if cfg.dtype == "f32":
                k[s, l], v[s, l] = post, vv
            else:
                k[s, l], v[s, l] = f32_to_bf16_bits(post), f32_to_bf16_bits(vv)
    return {"cfg": cfg, "k": k, "v": v, "pos": pos, "t": t, "qc": qc, "qn": qn, "rb": rb}


def make_device(cfg: Config, device="cuda", n_seq: int | None = None, n_layers: int | None = None,
                pre_rope: bool = False):
    """Draw a workload directly in device memory with torch (large configurations).

    Same recipe and layout as ``make_host``; K and V are torch tensors of dtype float32 or
    bfloat16 on ``device``.  Calibration statistics are drawn on the host (they are small).
    With ``pre_rope`` the cache holds the keys before RoPE.
    """
    import torch

    S = cfg.n_seq if n_seq is None else n_seq
    L = cfg.n_layers if n_layers is None else n_layers
    Hkv, N, d, h = cfg.n_kv_heads, cfg.n_keys, cfg.head_dim, cfg.head_dim // 2
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    qc, qn, rb = draw_calibration(rng, cfg, L)
    if cfg.t_fixed is not None:
        t = np.full(S, cfg.t_fixed, dtype=np.int32)
    else:
        t = rng.integers(cfg.t_range[0], cfg.t_range[1] + 1, size=S).astype(np.int32)
    kc = torch.from_numpy(8.0 * _unit(rng, (L, Hkv), d)).to(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    tdt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    k = torch.empty((S, L, Hkv, N, d), dtype=tdt, device=device)
    v = torch.empty((S, L, Hkv, N, d), dtype=tdt, device=device)
    pos = torch.empty((S, L, Hkv, N), dtype=torch.int32, device=device)
    w = torch.from_numpy(omega_table(d, cfg.theta)).to(device)
    for s in range(S):
        ts = int(t[s])
        if cfg.positions == "contiguous":
            p = torch.arange(ts - N + 1, ts + 1, dtype=torch.int64, device=device).expand(L, Hkv, N)
        else:
            n_old = N - 128
            r = torch.rand((L * Hkv, ts - 127), generator=gen, device=device)
            old = torch.sort(torch.argsort(r, dim=1)[:, :n_old], dim=1).values
            new = torch.arange(ts - 127, ts + 1, dtype=torch.int64, device=device).expand(L * Hkv, 128)
            p = torch.cat([old, new], dim=1).reshape(L, Hkv, N)
        pos[s] = p.to(torch.int32)
        for l in range(L):
            pre = kc[l][:, None, :] + 0.5 * torch.randn((Hkv, N, d), generator=gen, device=device,
                                                         dtype=torch.float64)
            if pre_rope:
                post = pre
            else:
                a = p[l].to(torch.float64)[..., None] * w
                c, sn = torch.cos(a), torch.sin(a)
                xr, xi = pre[..., :h], pre[..., h:]
                post = torch.cat([xr * c - xi * sn, xr * sn + xi * c], dim=-1)
                del a, c, sn
            k[s, l] = post.to(torch.float32).to(tdt)
            v[s, l] = torch.randn((Hkv, N, d), generator=gen, device=device).to(tdt)
            del pre, post
    t_dev = torch.from_numpy(t).to(device)
    return {"cfg": cfg, "k": k, "v": v, "pos": pos, "t": t, "t_dev": t_dev, "qc": qc, "qn": qn, "rb": rb}


def algorithmic_bytes(cfg: Config, moved_rows: int | None = None) -> int:
    """Bytes the prune step must move: K read once, the final score written and read once, and
    for every moved row its K and V rows read and written plus its position read and written."""
    r = cfg.head_dim * cfg.elem_bytes
    N = cfg.n_keys
    M = min(cfg.budget, N) * cfg.n_streams if moved_rows is None else moved_rows
    return cfg.n_streams * (N * r + 8 * N) + M * (4 * r + 8)


def to_device(wl: dict, device="cuda") -> dict:
    """Upload a host workload (``make_host``) to device tensors (same keys, torch tensors)."""
    import torch

    cfg = wl["cfg"]

    def cache(a):
        if cfg.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    out = dict(wl)
    out["k"] = cache(wl["k"])
    out["v"] = cache(wl["v"])
    out["pos"] = torch.from_numpy(np.ascontiguousarray(wl["pos"])).to(device)
    out["t_dev"] = torch.from_numpy(np.ascontiguousarray(wl["t"], dtype=np.int32)).to(device)
    return out


def cache_to_host(x) -> np.ndarray:
    """Device cache tensor -> numpy (float32, or uint16 bf16 bit patterns)."""
    import torch

    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()
