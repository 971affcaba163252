"""The streaming device copy (tria_copy; instrumentation, the read + write reference rate):
bytes copied exactly, nothing written past the end, sizes from one 16-byte word to more than the
capped grid covers in one stride."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 16 * (2048 * 3 + 7), 600 << 20])
def test_copy_is_exact(nbytes):
    import torch
    import kv_cache_compression_tria_amd as T
    print(f"\n[case] copy {nbytes} B", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(nbytes % 9973)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)
    full = torch.zeros(nbytes + 4096, dtype=torch.uint8, device="cuda")
    dst = full[:nbytes]
    T.copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert int(full[nbytes:].count_nonzero()) == 0


def test_copy_rejects_mismatched_sizes():
    import torch
    import kv_cache_compression_tria_amd as T
    a = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        T.copy(a, torch.zeros(80, dtype=torch.uint8, device="cuda"))
    with pytest.raises(T.TriaError):
        T.copy(a[:40], torch.zeros(40, dtype=torch.uint8, device="cuda"))
