"""TriAttention KV-cache prune step on AMD MI355X: thin Python binding over ``libtria.so``.

Every step of the prune path runs in the HIP kernels behind the C ABI declared in
``include/tria.h``; this module only marshals arguments (torch tensors give device pointers
and the current HIP stream).  If the library is missing, every call raises -- there is no
fallback path.

Entry points (same names as the C ABI, without the ``tria_`` prefix):
    load_calib, score, score_check, select_topB, compact, prune
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtria.so")

OK, E_INVALID, E_UNSUPPORTED, E_NOMEM, E_DEVICE, E_NONFINITE, E_WORKSPACE = 0, -1, -2, -3, -4, -5, -6
BF16, F32 = 0, 1
PER_KEY_PHASE = 1
KEYS_PRE_ROPE = 2
TRIG_WEIGHT_R = 4
OFFSET_MAX = 8
SCORE_TILED = 16

EXPORTED = (
    "tria_load_calib", "tria_free_calib", "tria_calib_dim", "tria_score_workspace_bytes", "tria_score",
    "tria_score_check", "tria_select_workspace_bytes", "tria_select_topB", "tria_compact",
    "tria_prune_workspace_bytes", "tria_prune", "tria_status_string", "tria_timing_enable", "tria_timing_read",
    "tria_calib_stats", "tria_append", "tria_decode_step", "tria_prune_static", "tria_band_tables", "tria_copy",
)
TIMERS = ("score_keys", "normalise", "select", "compact", "calib", "select_compact")


class TriaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtria.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # One HIP runtime per process: torch ships its own copy of the runtime libraries.  Loading
        # torch first makes libtria.so bind to that copy; loaded the other way round, the second
        # runtime to initialise finds no device.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_compression_tria_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, U, S, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_size_t, ctypes.c_double
        L.tria_load_calib.restype = I
        L.tria_load_calib.argtypes = [ctypes.POINTER(P), I, I, I, I, P, P, P, D, P, I, P]
        L.tria_free_calib.restype = None
        L.tria_free_calib.argtypes = [P]
        L.tria_calib_dim.restype = I
        L.tria_calib_dim.argtypes = [P, I]
        L.tria_score_workspace_bytes.restype = S
        L.tria_score_workspace_bytes.argtypes = [P, I, I, I, U]
        L.tria_score.restype = I
        L.tria_score.argtypes = [P, I, P, P, P, I, I, P, P, P, U, P, S, P]
        L.tria_score_check.restype = I
        L.tria_score_check.argtypes = [P, S, P]
        L.tria_select_workspace_bytes.restype = S
        L.tria_select_workspace_bytes.argtypes = [I, I, I]
        L.tria_select_topB.restype = I
        L.tria_select_topB.argtypes = [P, I, I, I, P, P, S, P]
        L.tria_compact.restype = I
        L.tria_compact.argtypes = [I, P, P, P, P, I, I, I, I, P]
        L.tria_prune_workspace_bytes.restype = S
        L.tria_prune_workspace_bytes.argtypes = [P, I, I, I, I, U]
        L.tria_prune.restype = I
        L.tria_prune.argtypes = [P, I, P, P, P, P, I, I, I, P, P, U, P, S, P]
        L.tria_status_string.restype = ctypes.c_char_p
        L.tria_status_string.argtypes = [I]
        L.tria_timing_enable.restype = I
        L.tria_timing_enable.argtypes = [I]
        L.tria_calib_stats.restype = I
        L.tria_append.restype = I
        L.tria_append.argtypes = [I, P, P, P, I, I, I, P, P, P, I, I, P]
        L.tria_decode_step.restype = I
        L.tria_decode_step.argtypes = [P, I, P, P, P, P, I, I, I, I, P, P, P, I, P, P, U, P, S,
                                       ctypes.POINTER(I), P]
        L.tria_calib_stats.argtypes = [I, P, I, I, I, I, P, P, P, P]
        L.tria_band_tables.restype = I
        L.tria_band_tables.argtypes = [D, I, P, I, P, P, P, P]
        L.tria_prune_static.restype = I
        L.tria_prune_static.argtypes = [P, I, P, P, P, P, I, I, I, P, P, U, ctypes.POINTER(P), P]
        L.tria_timing_read.restype = I
        L.tria_timing_read.argtypes = [ctypes.POINTER(D), ctypes.POINTER(I)]
        L.tria_copy.restype = I
        L.tria_copy.argtypes = [P, P, S, P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    try:
        return lib().tria_status_string(int(status)).decode()
    except Exception:  # library not loadable: still format the error
        return "status"


def _check(status: int, what: str):
    if status != OK:
        raise TriaError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported cache dtype {t.dtype}")


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Calib:
    """Handle of a device calibration table (``tria_load_calib``)."""

    def __init__(self, handle: ctypes.c_void_p, n_layers, n_q_heads, n_kv_heads):
        self._h = handle
        self.n_layers, self.n_q_heads, self.n_kv_heads = n_layers, n_q_heads, n_kv_heads
        self.G = n_q_heads // n_kv_heads

    @property
    def handle(self):
        return self._h

    def free(self):
        if self._h is not None and self._h.value:
            lib().tria_free_calib(self._h)
        self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def band_tables(rope_theta: float = 1e6, head_dim: int = 128, offsets=None):
    """Host-only per-band constants (``tria_band_tables``): (w, C, S, nu) as numpy arrays of
    head_dim/2 elements (float64, float64, float64, uint64)."""
    h = head_dim // 2
    w, C, S = (np.zeros(h, dtype=np.float64) for _ in range(3))
    nu = np.zeros(h, dtype=np.uint64)
    off = None if offsets is None else np.ascontiguousarray(offsets, dtype=np.int32)
    _check(lib().tria_band_tables(float(rope_theta), int(head_dim), None if off is None else off.ctypes.data,
                                  0 if off is None else len(off), w.ctypes.data, C.ctypes.data, S.ctypes.data,
                                  nu.ctypes.data), "tria_band_tables")
    return w, C, S, nu


def load_calib(q_centre, q_band_norm, r_band, n_kv_heads: int, rope_theta: float = 1e6,
               offsets=None, stream=None) -> Calib:
    """q_centre [L][Hq][d], q_band_norm / r_band [L][Hq][d/2] (host arrays, float32)."""
    qc = np.ascontiguousarray(q_centre, dtype=np.float32)
    qn = np.ascontiguousarray(q_band_norm, dtype=np.float32)
    rb = np.ascontiguousarray(r_band, dtype=np.float32)
    if qc.ndim != 3:
        raise ValueError("q_centre must be [L][Hq][d]")
    L, Hq, d = qc.shape
    if qn.shape != (L, Hq, d // 2) or rb.shape != (L, Hq, d // 2):
        raise ValueError("q_band_norm and r_band must be [L][Hq][d/2]")
    off = None if offsets is None else np.ascontiguousarray(offsets, dtype=np.int32)
    h = ctypes.c_void_p()
    st = lib().tria_load_calib(ctypes.byref(h), L, Hq, int(n_kv_heads), d, qc.ctypes.data, qn.ctypes.data,
                               rb.ctypes.data, float(rope_theta), None if off is None else off.ctypes.data,
                               0 if off is None else len(off), _stream(stream))
    _check(st, "tria_load_calib")
    return Calib(h, L, Hq, int(n_kv_heads))


def _dtype_arg(dtype) -> int:
    import torch
    if dtype in (BF16, F32):
        return int(dtype)
    if dtype == torch.bfloat16:
        return BF16
    if dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported cache dtype {dtype}")


def score_workspace_bytes(calib: Calib, n_seq: int, n_keys: int, dtype=BF16, flags: int = 0) -> int:
    """Workspace bytes of ``score`` with these flags (``tria_score_workspace_bytes``)."""
    return int(lib().tria_score_workspace_bytes(calib.handle, _dtype_arg(dtype), int(n_seq), int(n_keys), int(flags)))


def workspace(nbytes: int, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def score(calib: Calib, k, t, F=None, raw=None, head_stats=None, pos=None, flags: int = 0, ws=None,
          stream=None, check: bool = False):
    """Final scores F [S][L][Hkv][N] of every key (``tria_score``).

    k [S][L][Hkv][N][128] (bf16 or fp32), t [S] int32 on the device; optional raw
    [S][L][Hq][N] and head_stats [S][L][Hq][2] float32 outputs.
    """
    import torch
    S, L, Hkv, N, d = k.shape
    for name, x in (("k", k), ("t", t), ("F", F), ("raw", raw), ("head_stats", head_stats), ("pos", pos)):
        _dev(x, name)
    if F is None:
        F = torch.empty((S, L, Hkv, N), dtype=torch.float32, device=k.device)
    if ws is None:
        ws = workspace(score_workspace_bytes(calib, S, N, k.dtype, flags), k.device)
    st = lib().tria_score(calib.handle, _dtype_code(k), _ptr(k), _ptr(pos), _ptr(t), S, N, _ptr(F), _ptr(raw),
                          _ptr(head_stats), int(flags), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream(stream))
    _check(st, "tria_score")
    if check:
        score_check(ws, stream)
    return F


def score_check(ws, stream=None):
    _check(lib().tria_score_check(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "tria_score")


def select_topB(F, budget: int, kept=None, stream=None):
    """kept [streams][min(B,N)] int32, ascending (``tria_select_topB``)."""
    import torch
    _dev(F, "F")
    N = F.shape[-1]
    n_streams = F.numel() // N
    nk = min(int(budget), N)
    if kept is None:
        kept = torch.empty((n_streams, nk), dtype=torch.int32, device=F.device)
    _dev(kept, "kept")
    nb = int(lib().tria_select_workspace_bytes(n_streams, N, int(budget)))
    ws = workspace(nb, F.device)
    _check(lib().tria_select_topB(_ptr(F), n_streams, N, int(budget), _ptr(kept), _ptr(ws), ws.numel(),
                                  _stream(stream)), "tria_select_topB")
    return kept


def compact(k, v, pos, kept, budget: int, stream=None):
    """In-place compaction of K, V (and pos) by kept (``tria_compact``)."""
    for name, x in (("k", k), ("v", v), ("pos", pos), ("kept", kept)):
        _dev(x, name)
    N, d = k.shape[-2], k.shape[-1]
    n_streams = k.numel() // (N * d)
    _check(lib().tria_compact(_dtype_code(k), _ptr(k), _ptr(v), _ptr(pos), _ptr(kept), n_streams, N, int(budget),
                              d, _stream(stream)), "tria_compact")


def prune_workspace_bytes(calib: Calib, n_seq: int, n_keys: int, budget: int, dtype=BF16, flags: int = 0) -> int:
    """Workspace bytes of ``prune`` / ``decode_step`` with these flags (``tria_prune_workspace_bytes``)."""
    return int(lib().tria_prune_workspace_bytes(calib.handle, _dtype_arg(dtype), int(n_seq), int(n_keys),
                                                int(budget), int(flags)))


def prune(calib: Calib, k, v, pos, t, budget: int, F=None, kept=None, flags: int = 0, ws=None, stream=None,
          check: bool = True):
    """Whole prune step (``tria_prune``): returns (F, kept); K, V, pos compacted in place.

    With ``check`` (the default) the call waits for the step and raises if the scoring failed on
    the device (``tria_score_check``; K, V and pos are then left as they were).  Without it the
    call stays asynchronous and the caller checks ``ws`` itself."""
    import torch
    S, L, Hkv, N, d = k.shape
    for name, x in (("k", k), ("v", v), ("pos", pos), ("t", t), ("F", F), ("kept", kept)):
        _dev(x, name)
    if F is None:
        F = torch.empty((S, L, Hkv, N), dtype=torch.float32, device=k.device)
    if kept is None:
        kept = torch.empty((S * L * Hkv, min(int(budget), N)), dtype=torch.int32, device=k.device)
    if ws is None:
        ws = workspace(prune_workspace_bytes(calib, S, N, budget, k.dtype, flags), k.device)
    st = lib().tria_prune(calib.handle, _dtype_code(k), _ptr(k), _ptr(v), _ptr(pos), _ptr(t), S, N, int(budget),
                          _ptr(F), _ptr(kept), int(flags), _ptr(ws), ws.numel() * ws.element_size(),
                          _stream(stream))
    _check(st, "tria_prune")
    if check:
        score_check(ws, stream)
    return F, kept


STATIC_WORKSPACE_BYTES = 64 << 20


def prune_static(calib: Calib, k, v, pos, t, budget: int, F=None, kept=None, flags: int = 0, stream=None,
                 check: bool = True):
    """The prune step without a caller workspace (``tria_prune_static``): the library's static
    device array of STATIC_WORKSPACE_BYTES serves as scratch, so the call allocates nothing (F and
    kept must then be passed in by a caller that cannot allocate).  Returns (F, kept, ws_addr);
    ws_addr is the device address of that array, for ``score_check_addr``.  With ``check`` (the
    default) the call waits for the step and raises if the scoring failed on the device."""
    import torch
    S, L, Hkv, N, d = k.shape
    for name, x in (("k", k), ("v", v), ("pos", pos), ("t", t), ("F", F), ("kept", kept)):
        _dev(x, name)
    if F is None:
        F = torch.empty((S, L, Hkv, N), dtype=torch.float32, device=k.device)
    if kept is None:
        kept = torch.empty((S * L * Hkv, min(int(budget), N)), dtype=torch.int32, device=k.device)
    addr = ctypes.c_void_p()
    st = lib().tria_prune_static(calib.handle, _dtype_code(k), _ptr(k), _ptr(v), _ptr(pos), _ptr(t), S, N,
                                 int(budget), _ptr(F), _ptr(kept), int(flags), ctypes.byref(addr), _stream(stream))
    _check(st, "tria_prune_static")
    if check:
        score_check_addr(addr.value, stream)
    return F, kept, addr.value


def score_check_addr(ws_addr: int, stream=None):
    """``tria_score_check`` on a workspace given by its device address (as ``prune_static`` returns)."""
    _check(lib().tria_score_check(ctypes.c_void_p(ws_addr), 256, _stream(stream)), "tria_score")


def calib_stats(q, q_centre=None, q_band_norm=None, r_band=None, stream=None):
    """Calibration statistics of captured pre-RoPE queries q [L][Hq][n_cal][128] (bf16 or fp32)
    on the device (``tria_calib_stats``): returns (q_centre [L][Hq][128], q_band_norm [L][Hq][64],
    r_band [L][Hq][64]) float32 device tensors, the inputs of ``load_calib``."""
    import torch
    _dev(q, "q")
    L, Hq, n_cal, d = q.shape
    outs = []
    for x, shape in ((q_centre, (L, Hq, d)), (q_band_norm, (L, Hq, d // 2)), (r_band, (L, Hq, d // 2))):
        if x is None:
            x = torch.empty(shape, dtype=torch.float32, device=q.device)
        _dev(x, "output")
        outs.append(x)
    _check(lib().tria_calib_stats(_dtype_code(q), _ptr(q), L, Hq, n_cal, d, _ptr(outs[0]), _ptr(outs[1]),
                                  _ptr(outs[2]), _stream(stream)), "tria_calib_stats")
    return tuple(outs)


def append(k, v, pos, length: int, k_new, v_new, pos_new, stream=None):
    """Copy the new rows k_new/v_new [S][L][Hkv][n][d] and pos_new [S][L][Hkv][n] into rows
    [length, length + n) of the cache k/v [S][L][Hkv][cap][d], pos [S][L][Hkv][cap]
    (``tria_append``)."""
    S, L, Hkv, cap, d = k.shape
    n = k_new.shape[-2]
    for name, x in (("k", k), ("v", v), ("pos", pos), ("k_new", k_new), ("v_new", v_new), ("pos_new", pos_new)):
        _dev(x, name)
    _check(lib().tria_append(_dtype_code(k), _ptr(k), _ptr(v), _ptr(pos), S * L * Hkv, cap, int(length), _ptr(k_new),
                             _ptr(v_new), _ptr(pos_new), n, d, _stream(stream)), "tria_append")


def decode_step(calib: Calib, k, v, pos, t, length: int, budget: int, k_new, v_new, pos_new, F=None, kept=None,
                flags: int = 0, ws=None, stream=None, check: bool = True) -> int:
    """Append the new rows and, when that fills the cache, prune it back to ``budget`` rows
    (``tria_decode_step``).  Returns the live length afterwards.  With ``check`` (the default) a
    step that pruned waits for the device and raises if the scoring failed (the cache is then
    left unpruned, cap rows live)."""
    import torch
    S, L, Hkv, cap, d = k.shape
    n = k_new.shape[-2]
    for name, x in (("k", k), ("v", v), ("pos", pos), ("t", t), ("k_new", k_new), ("v_new", v_new),
                    ("pos_new", pos_new), ("F", F), ("kept", kept)):
        _dev(x, name)
    if F is None:
        F = torch.empty((S, L, Hkv, cap), dtype=torch.float32, device=k.device)
    if kept is None:
        kept = torch.empty((S * L * Hkv, min(int(budget), cap)), dtype=torch.int32, device=k.device)
    if ws is None:
        ws = workspace(prune_workspace_bytes(calib, S, cap, budget, k.dtype, flags), k.device)
    out = ctypes.c_int(0)
    _check(lib().tria_decode_step(calib.handle, _dtype_code(k), _ptr(k), _ptr(v), _ptr(pos), _ptr(t), S, cap,
                                  int(length), int(budget), _ptr(k_new), _ptr(v_new), _ptr(pos_new), n, _ptr(F),
                                  _ptr(kept), int(flags), _ptr(ws), ws.numel() * ws.element_size(),
                                  ctypes.byref(out), _stream(stream)), "tria_decode_step")
    if check and int(length) + n == cap and cap > int(budget):
        score_check(ws, stream)
    return out.value


def timing_enable(on: bool = True):
    """Turn per-kernel event timing on or off (``tria_timing_enable``)."""
    _check(lib().tria_timing_enable(1 if on else 0), "tria_timing_enable")


def copy(src, dst, stream=None):
    """Streaming device copy of src into dst (``tria_copy``; instrumentation: the read + write
    reference rate).  Both contiguous device tensors of the same byte size, a multiple of 16."""
    if src is None or dst is None:
        raise ValueError("copy: src and dst are required")
    for name, x in (("src", src), ("dst", dst)):
        _dev(x, name)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("copy: src and dst differ in size")
    _check(lib().tria_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)), "tria_copy")


def timing_read() -> dict:
    """Summed milliseconds and launch counts per timed kernel since the last read
    (``tria_timing_read``); waits for the recorded events."""
    ms = (ctypes.c_double * len(TIMERS))()
    n = (ctypes.c_int * len(TIMERS))()
    _check(lib().tria_timing_read(ms, n), "tria_timing_read")
    return {name: {"ms": ms[i], "launches": n[i]} for i, name in enumerate(TIMERS)}
