"""Top-B selection on the GPU against the oracle's full sort, on hand-made score rows.

The selection brackets the threshold from a strided sample of the scores and falls back to a
radix selection over all keys when the bracket misses; these rows exercise both routes (sample
ranges that miss, heavy ties, a sampled outlier, constant rows) in both bracketed kernels (the
one that streams F for 8193-32768 keys, the one that copies short streams to LDS), the global
kernel past 32768 keys, and the edges of B.  Every result is
compared bit-exactly with the oracle's selection on the same float32 scores (ties to the lower
index, output ascending).
"""
import numpy as np
import pytest

from oracle import oracle as orc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    import kv_cache_compression_tria_amd as T
    T.lib()
    return T


def _select(T, F, B):
    import torch
    Fd = torch.from_numpy(np.ascontiguousarray(F, dtype=np.float32)).to("cuda")
    kept = T.select_topB(Fd, B)
    torch.cuda.synchronize()
    return kept.cpu().numpy()


def _check(T, F, B):
    F = np.ascontiguousarray(F, dtype=np.float32)
    kept = _select(T, F, B)
    for i in range(F.shape[0]):
        ref = orc.select(F[i].astype(np.float64), B)
        assert np.array_equal(kept[i], ref), f"row {i}: selection differs from the oracle's full sort"


def _rows(rng, n, N):
    # maxima of eight normal z-scores, the shape of final scores
    return rng.standard_normal((n, N, 8)).max(axis=2).astype(np.float32)


@pytest.mark.parametrize("N,B", [(32768, 3072), (2176, 2048), (8192, 900), (8193, 4000), (30001, 17)])
def test_score_like_rows(T, N, B):
    rng = np.random.default_rng(N + B)
    _check(T, _rows(rng, 6, N), B)


@pytest.mark.parametrize("N,B", [(32768, 1), (32768, 32767), (2176, 1), (2176, 2175), (640, 320)])
def test_budget_edges(T, N, B):
    rng = np.random.default_rng(7 * N + B)
    _check(T, _rows(rng, 3, N), B)


def test_sample_misses_the_threshold(T):
    """The strided sample sees only low scores while every other key is high: the bracket from the
    sample cannot hold the threshold and the fallback must decide."""
    rng = np.random.default_rng(11)
    for N, B in ((32768, 3072), (2176, 2048)):
        nt = 1024 if N > 8192 else 256
        stride = N // min(N, nt)
        F = (1.0 + rng.random((2, N))).astype(np.float32)
        F[:, ::stride] = -rng.random((2, len(range(0, N, stride))))
        _check(T, F, B)


def test_heavy_ties(T):
    rng = np.random.default_rng(12)
    F = np.round(rng.standard_normal((4, 32768)) * 2.0) / 2.0          # nine distinct values
    _check(T, F, 3072)
    F = np.round(rng.standard_normal((4, 2176)) * 2.0) / 2.0
    _check(T, F, 2048)


def test_constant_rows_keep_the_prefix(T):
    F = np.zeros((2, 32768), dtype=np.float32)
    F[1] = 1.5
    kept = _select(T, F, 3072)
    assert np.array_equal(kept, np.tile(np.arange(3072), (2, 1)))


def test_sampled_outlier_widens_the_bracket(T):
    """One huge sampled score stretches the sample's linear bins: the bracket holds far more keys
    than the candidate list and the fallback must decide."""
    rng = np.random.default_rng(13)
    F = _rows(rng, 2, 32768)
    F[:, 0] = 1.0e30
    _check(T, F, 3072)


def test_signed_zeros_and_negative_rows(T):
    rng = np.random.default_rng(14)
    F = -np.abs(_rows(rng, 2, 32768))
    F[0, ::3] = 0.0
    F[0, 1::3] = -0.0
    _check(T, F, 3072)


def test_past_the_lds_limit(T):
    rng = np.random.default_rng(15)
    _check(T, _rows(rng, 2, 40000), 3000)


def test_library_loaded_before_torch_touches_the_gpu():
    """The library is loaded before torch initialises the GPU (a fresh process): the binding
    loads torch's HIP runtime first, so the selection still runs."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import kv_cache_compression_tria_amd as T\n"
            "T.lib()\n"
            "import torch\n"
            "F = torch.arange(4096, dtype=torch.float32, device='cuda').reshape(2, 2048)\n"
            "k = T.select_topB(F, 100)\n"
            "torch.cuda.synchronize()\n"
            "assert k.cpu().tolist() == [list(range(1948, 2048))] * 2\n"
            "print('ok')\n") % root
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
