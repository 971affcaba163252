"""ctypes wrapper around the fp64 C oracle (``tria_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of the benchmark
use this module.  The product library never imports it, and it imports nothing from the
product library.  See ``tria_oracle.c`` for what is computed and which page each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tria_oracle.c")
_LIB = os.path.join(_HERE, "libtria_oracle.so")

DEFAULT_OFFSETS = tuple(2 ** i for i in range(17))  # D = {1, 2, 4, ..., 2^16}
_FORMS = {"lit": 0, "fac": 1, "max": 2}            # offset mean (literal / factored), offset max


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        L.oracle_omega.restype = D
        L.oracle_omega.argtypes = [D, I, I]
        L.oracle_score_stream.restype = None
        L.oracle_score_stream.argtypes = [I, I, I, I, P, P, ctypes.c_int64, P, P, P, D, P, I, I, I, I, P, P, P]
        L.oracle_zmax.restype = I
        L.oracle_zmax.argtypes = [I, I, P, P, P, P, P]
        L.oracle_select.restype = I
        L.oracle_select.argtypes = [I, I, P, P]
        L.oracle_compact_rows.restype = None
        L.oracle_compact_rows.argtypes = [I, ctypes.c_size_t, P, P]
        L.oracle_prune_streams.restype = I
        L.oracle_prune_streams.argtypes = [I, I, I, I, I, I, I, I, I, I, P, P, P, P, P, P, D, P, I, I,
                                           P, I, P, P, P, I]
        L.oracle_calib_stats.restype = None
        L.oracle_calib_stats.argtypes = [I, I, I, I, P, P, P, P]
        L.oracle_max_threads.restype = I
        L.oracle_max_threads.argtypes = [I]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _keys_dtype(keys: np.ndarray) -> int:
    if keys.dtype == np.uint16:
        return 0  # bf16 bit patterns
    if keys.dtype == np.float32:
        return 1
    raise TypeError("keys must be bf16 bits (uint16) or float32")


def omega(theta: float, f: int, d: int) -> float:
    return lib().oracle_omega(theta, f, d)


def score_stream(keys, pos, t, qc, qn, rb, theta=1e6, offsets=DEFAULT_OFFSETS, form="lit", pre_rope=False,
                 weight_r=False):
    """Raw scores of one stream.

    keys [N][d] (uint16 bf16 bits or float32; post-RoPE, or pre-RoPE with ``pre_rope``),
    pos [N] int32, t int,
    qc [G][d], qn [G][d/2], rb [G][d/2] float32.
    Returns (s_trig, s_norm, raw), each float64 [G][N].
    """
    keys = np.ascontiguousarray(keys)
    N, d = keys.shape
    qc = np.ascontiguousarray(qc, dtype=np.float32).reshape(-1, d)
    G = qc.shape[0]
    qn = np.ascontiguousarray(qn, dtype=np.float32).reshape(G, d // 2)
    rb = np.ascontiguousarray(rb, dtype=np.float32).reshape(G, d // 2)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    st = np.zeros((G, N))
    sn = np.zeros((G, N))
    raw = np.zeros((G, N))
    lib().oracle_score_stream(N, d, G, _keys_dtype(keys), _ptr(keys), _ptr(pos), int(t), _ptr(qc),
                              _ptr(qn), _ptr(rb), float(theta), _ptr(off), len(off),
                              _FORMS[form], int(bool(pre_rope)), int(bool(weight_r)), _ptr(st),
                              _ptr(sn), _ptr(raw))
    return st, sn, raw


def zmax(raw):
    """raw [G][N] float64 -> (z [G][N], F [N], mu [G], sd [G])."""
    raw = np.ascontiguousarray(raw, dtype=np.float64)
    G, N = raw.shape
    z = np.zeros((G, N))
    F = np.zeros(N)
    mu = np.zeros(G)
    sd = np.zeros(G)
    rc = lib().oracle_zmax(N, G, _ptr(raw), _ptr(z), _ptr(F), _ptr(mu), _ptr(sd))
    if rc != 0:
        raise ValueError("non-finite raw score")
    return z, F, mu, sd


def select(F, B):
    """Top-B of F by (F desc, index asc), returned ascending (int32)."""
    F = np.ascontiguousarray(F, dtype=np.float64)
    N = F.shape[0]
    kept = np.zeros(max(min(B, N), 1), dtype=np.int32)
    n = lib().oracle_select(N, int(B), _ptr(F), _ptr(kept))
    if n < 0:
        raise ValueError("non-finite score")
    return kept[:n]


def compact_rows(rows: np.ndarray, kept: np.ndarray) -> np.ndarray:
    """Out-of-place reference compaction: returns a copy with row i <- row kept[i] for i < len(kept)."""
    out = np.ascontiguousarray(rows).copy()
    kept = np.ascontiguousarray(kept, dtype=np.int32)
    row_bytes = out.nbytes // out.shape[0]
    lib().oracle_compact_rows(len(kept), row_bytes, _ptr(out), _ptr(kept))
    return out


def prune_streams(keys, pos, t, qc, qn, rb, B, n_kv_heads, stream_ids=None, theta=1e6,
                  offsets=DEFAULT_OFFSETS, form="fac", want_raw=False, n_threads=0, pre_rope=False, weight_r=False):
    """Oracle prune over a list of streams.

    keys [n][N][d] and pos [n][N] hold the listed streams (packed, in ``stream_ids`` order);
    keys are post-RoPE, or the pre-RoPE bands themselves with ``pre_rope``; ``weight_r`` weights
    each band's trigonometric term by R_f;
    ``stream_ids`` are the global ids (s*L + l)*Hkv + g (default: 0..n-1).
    t [S], qc [L][Hq][d], qn/rb [L][Hq][d/2].
    Returns dict with F [n][N], kept [n][min(B,N)] and (optionally) raw [n][G][N].
    """
    keys = np.ascontiguousarray(keys)
    d = keys.shape[-1]
    N = keys.shape[-2]
    keys = keys.reshape(-1, N, d)
    n = keys.shape[0]
    L, Hq = qc.shape[0], qc.shape[1]
    Hkv = int(n_kv_heads)
    G = Hq // Hkv
    S = int(np.asarray(t).size)
    if stream_ids is None:
        stream_ids = np.arange(n)
    ids = np.ascontiguousarray(stream_ids, dtype=np.int64)
    assert len(ids) == n
    nk = min(B, N)
    F = np.zeros((n, N))
    kept = np.zeros((n, nk), dtype=np.int32)
    raw = np.zeros((n, G, N)) if want_raw else None
    # keep every converted array bound to a name for the duration of the call
    tt = np.ascontiguousarray(t, dtype=np.int64).reshape(S)
    pp = np.ascontiguousarray(pos, dtype=np.int32)
    qc_ = np.ascontiguousarray(qc, dtype=np.float32)
    qn_ = np.ascontiguousarray(qn, dtype=np.float32)
    rb_ = np.ascontiguousarray(rb, dtype=np.float32)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    rc = lib().oracle_prune_streams(_FORMS[form], int(bool(pre_rope)), int(bool(weight_r)), _keys_dtype(keys), S, L, Hkv, G, N, d,
                                    _ptr(keys), _ptr(pp), _ptr(tt), _ptr(qc_), _ptr(qn_), _ptr(rb_),
                                    float(theta), _ptr(off), len(off), int(B), _ptr(ids), n,
                                    _ptr(F), _ptr(raw), _ptr(kept), int(n_threads))
    if rc != 0:
        raise ValueError("non-finite score")
    out = {"F": F, "kept": kept}
    if want_raw:
        out["raw"] = raw
    return out


def calib_stats(q):
    """Calibration statistics of captured pre-RoPE queries q [..., n_cal, d] (uint16 bf16 bits or
    float32): returns (qbar [..., d], E|q_f| [..., d/2], R_f [..., d/2]) in float64."""
    q = np.ascontiguousarray(q)
    d, n_cal = q.shape[-1], q.shape[-2]
    lead = q.shape[:-2]
    n_heads = int(np.prod(lead)) if lead else 1
    qc = np.zeros(lead + (d,))
    qn = np.zeros(lead + (d // 2,))
    r = np.zeros(lead + (d // 2,))
    lib().oracle_calib_stats(n_heads, n_cal, d, _keys_dtype(q), _ptr(q), _ptr(qc), _ptr(qn), _ptr(r))
    return qc, qn, r


def max_threads(n_threads: int = 0) -> int:
    return lib().oracle_max_threads(int(n_threads))
