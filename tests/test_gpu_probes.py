"""The measurement probes behind bench.py's measured peaks: the copy moves
every byte (a copy of random bytes equals its source, the bytes past it are
untouched), and the matrix-core loop runs and returns finite sums with the
stated FLOP count."""
import pytest
import torch

from combine_wave_level_amd import moe

pytestmark = pytest.mark.gpu


def test_copy_probe_copies_exactly():
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    n = (64 << 20) + 48
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.full((n + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    moe.probe_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert (dst[n:] == 0xA5).all()


def test_mfma_probe_runs_and_counts_flops():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out, flops = moe.probe_mfma(64)
    torch.cuda.synchronize()
    assert flops == cus * 8 * 64 * 16 * (2 * 16 * 16 * 32)
    assert out.numel() == cus * 512 and torch.isfinite(out).all()
    with pytest.raises(moe.MoEError):
        moe.probe_mfma(64, out=out[: cus * 512 - 1])
