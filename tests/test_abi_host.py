"""Host-side checks of the C-ABI library (CPU only: no kernel is launched).

* libtria.so loads and exports every function declared in include/tria.h;
* argument validation returns its documented status before touching the device.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tria.h")


@pytest.fixture(scope="module")
def tria():
    import kv_cache_compression_tria_amd as T
    if not os.path.exists(T.LIB_PATH):
        from kv_cache_compression_tria_amd import build
        build.build()
    return T


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tria_[A-Za-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("tria_load_calib", "tria_score", "tria_select_topB", "tria_compact"):
        assert required in names


def test_library_exports_every_declared_symbol(tria):
    L = tria.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(tria.EXPORTED)


def test_status_strings(tria):
    L = tria.lib()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.tria_status_string(code).decode() not in ("", "unknown status")
    assert L.tria_status_string(7).decode() == "unknown status"


def _calib_args(L=1, Hq=4, Hkv=1, d=128):
    qc = np.ones((L, Hq, d), np.float32)
    qn = np.ones((L, Hq, d // 2), np.float32)
    rb = np.full((L, Hq, d // 2), 0.9, np.float32)
    return qc, qn, rb


def test_load_calib_validation(tria):
    L = tria.lib()
    h = ctypes.c_void_p()
    qc, qn, rb = _calib_args()
    P = lambda a: a.ctypes.data
    assert L.tria_load_calib(None, 1, 4, 1, 128, P(qc), P(qn), P(rb), 1e6, None, 0, None) == tria.E_INVALID
    assert L.tria_load_calib(ctypes.byref(h), 1, 4, 1, 128, None, P(qn), P(rb), 1e6, None, 0, None) == tria.E_INVALID
    assert L.tria_load_calib(ctypes.byref(h), 0, 4, 1, 128, P(qc), P(qn), P(rb), 1e6, None, 0, None) == tria.E_INVALID
    assert L.tria_load_calib(ctypes.byref(h), 1, 4, 1, 128, P(qc), P(qn), P(rb), 0.5, None, 0, None) == tria.E_INVALID
    qc64, qn64, rb64 = _calib_args(d=64)
    assert L.tria_load_calib(ctypes.byref(h), 1, 4, 1, 64, P(qc64), P(qn64), P(rb64), 1e6, None, 0,
                             None) == tria.E_UNSUPPORTED
    assert L.tria_load_calib(ctypes.byref(h), 1, 6, 4, 128, P(qc), P(qn), P(rb), 1e6, None, 0,
                             None) == tria.E_UNSUPPORTED                 # Hq not a multiple of Hkv
    qc16, qn16, rb16 = _calib_args(Hq=16)
    assert L.tria_load_calib(ctypes.byref(h), 1, 16, 1, 128, P(qc16), P(qn16), P(rb16), 1e6, None, 0,
                             None) == tria.E_UNSUPPORTED                 # G = 16 > 8
    bad_r = rb.copy()
    bad_r[0, 0, 3] = 1.5
    assert L.tria_load_calib(ctypes.byref(h), 1, 4, 1, 128, P(qc), P(qn), P(bad_r), 1e6, None, 0,
                             None) == tria.E_INVALID
    bad_q = qc.copy()
    bad_q[0, 1, 2] = np.nan
    assert L.tria_load_calib(ctypes.byref(h), 1, 4, 1, 128, P(bad_q), P(qn), P(rb), 1e6, None, 0,
                             None) == tria.E_INVALID
    off = np.array([1, -2], np.int32)
    assert L.tria_load_calib(ctypes.byref(h), 1, 4, 1, 128, P(qc), P(qn), P(rb), 1e6, P(off), 2,
                             None) == tria.E_INVALID
    assert L.tria_load_calib(ctypes.byref(h), 1, 4, 1, 128, P(qc), P(qn), P(rb), 1e6, None, 3,
                             None) == tria.E_INVALID


def test_score_select_compact_validation(tria):
    L = tria.lib()
    fake = ctypes.c_void_p(0x1000)    # never dereferenced: validation fails first
    assert L.tria_score(None, 0, fake, None, fake, 1, 16, fake, None, None, 0, fake, 1 << 20, None) == tria.E_INVALID
    assert L.tria_score_workspace_bytes(None, 0, 1, 16, 0) == 0
    assert L.tria_prune_workspace_bytes(None, 0, 1, 16, 8, 0) == 0
    assert L.tria_select_topB(None, 1, 16, 4, fake, fake, 256, None) == tria.E_INVALID
    assert L.tria_select_topB(fake, 1, 0, 4, fake, fake, 256, None) == tria.E_INVALID
    assert L.tria_select_topB(fake, 1, 16, 0, fake, fake, 256, None) == tria.E_INVALID
    assert L.tria_select_topB(fake, 1, 16, 4, fake, None, 0, None) == tria.E_WORKSPACE
    assert L.tria_compact(0, None, fake, None, fake, 1, 16, 4, 128, None) == tria.E_INVALID
    assert L.tria_compact(2, fake, fake, None, fake, 1, 16, 4, 128, None) == tria.E_INVALID
    assert L.tria_compact(0, fake, fake, None, fake, 1, 16, 4, 64, None) == tria.E_UNSUPPORTED
    assert L.tria_compact(0, ctypes.c_void_p(0x1001), fake, None, fake, 1, 16, 4, 128, None) == tria.E_INVALID
    # B >= N is the identity: nothing to launch
    assert L.tria_compact(0, fake, fake, None, fake, 1, 16, 16, 128, None) == tria.OK
    assert L.tria_prune(None, 0, fake, fake, None, fake, 1, 16, 4, fake, fake, 0, fake, 1 << 20, None) == tria.E_INVALID


def test_copy_validation(tria):
    """tria_copy refuses NULL, empty, ragged, misaligned and overlapping buffers before any launch."""
    L = tria.lib()
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)     # never dereferenced
    assert L.tria_copy(None, b, 1024, None) == tria.E_INVALID
    assert L.tria_copy(a, None, 1024, None) == tria.E_INVALID
    assert L.tria_copy(a, b, 0, None) == tria.E_INVALID
    assert L.tria_copy(a, b, 1000, None) == tria.E_INVALID
    assert L.tria_copy(ctypes.c_void_p(0x100008), b, 1024, None) == tria.E_INVALID
    assert L.tria_copy(a, ctypes.c_void_p(0x100000 + 512), 1024, None) == tria.E_INVALID
    assert L.tria_copy(ctypes.c_void_p(0x100000 + 512), a, 1024, None) == tria.E_INVALID


def test_timing_api_without_pending_events(tria):
    """Timing can be switched on and off and read with nothing recorded (no GPU needed)."""
    T = tria
    L = T.lib()
    nt = len(T.TIMERS)                  # TRIA_TIMER_COUNT
    ms = (ctypes.c_double * nt)()
    n = (ctypes.c_int * nt)()
    assert L.tria_timing_enable(1) == T.OK
    assert L.tria_timing_read(ms, n) == T.OK
    assert list(n) == [0] * nt and list(ms) == [0.0] * nt
    assert L.tria_timing_enable(0) == T.OK
    assert L.tria_timing_read(None, n) == T.E_INVALID
    assert T.timing_read() == {name: {"ms": 0.0, "launches": 0} for name in T.TIMERS}


def test_timer_names_match_header(tria):
    """The binding names one timer per TRIA_TIMER_* slot (tria_timing_read writes COUNT entries)."""
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "tria.h")).read()
    count = int(re.search(r"TRIA_TIMER_COUNT\s*=\s*(\d+)", text).group(1))
    assert len(tria.TIMERS) == count


def test_calib_append_decode_validation(tria):
    """Argument errors of the calibration, append and decode-step entry points are reported
    before any launch."""
    L = tria.lib()
    fake = ctypes.c_void_p(0x1000)
    # tria_calib_stats(dtype, q, L, Hq, n_cal, d, qc, qn, rb, stream)
    assert L.tria_calib_stats(0, None, 1, 1, 4, 128, fake, fake, fake, None) == tria.E_INVALID
    assert L.tria_calib_stats(0, fake, 1, 1, 0, 128, fake, fake, fake, None) == tria.E_INVALID
    assert L.tria_calib_stats(5, fake, 1, 1, 4, 128, fake, fake, fake, None) == tria.E_INVALID
    assert L.tria_calib_stats(0, fake, 1, 1, 4, 64, fake, fake, fake, None) == tria.E_UNSUPPORTED
    assert L.tria_calib_stats(0, ctypes.c_void_p(0x1008), 1, 1, 4, 128, fake, fake, fake, None) == tria.E_INVALID
    # tria_append(dtype, k, v, pos, n_streams, cap, len, kn, vn, pn, n_new, d, stream)
    assert L.tria_append(0, fake, fake, fake, 1, 16, 8, fake, fake, fake, 9, 128, None) == tria.E_INVALID   # overflow
    assert L.tria_append(0, fake, fake, fake, 1, 16, -1, fake, fake, fake, 4, 128, None) == tria.E_INVALID
    assert L.tria_append(0, fake, fake, fake, 1, 16, 0, fake, fake, fake, 0, 128, None) == tria.E_INVALID
    assert L.tria_append(0, fake, fake, fake, 1, 16, 0, fake, fake, None, 4, 128, None) == tria.E_INVALID  # pos w/o pos_new
    assert L.tria_append(0, fake, fake, None, 1, 16, 0, fake, fake, None, 4, 64, None) == tria.E_UNSUPPORTED
    assert L.tria_append(0, ctypes.c_void_p(0x1004), fake, None, 1, 16, 0, fake, fake, None, 4, 128, None) == tria.E_INVALID
    out = ctypes.c_int(-7)
    assert L.tria_decode_step(None, 0, fake, fake, fake, fake, 1, 16, 0, 8, fake, fake, fake, 4, fake, fake, 0,
                              fake, 1 << 20, ctypes.byref(out), None) == tria.E_INVALID
    assert out.value == -7
