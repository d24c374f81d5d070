"""GPU check of the streaming-read helper used for achievable-bandwidth
figures: the XOR of its per-workgroup words equals the XOR of every 32-bit
word of the buffer (so every byte was read, once)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

tidar = pytest.importorskip("diffusion_drafted_self_amd")
import torch  # noqa: E402


# the third size is the smallest that runs the eight-load loop (8 strides of 16384 x 256 pieces) plus a tail
@pytest.mark.parametrize("n_words", [4, 12, 16384 * 256 * 4 * 8 + 12, 3 * (1 << 20) + 4])
def test_read_probe_folds_every_word(n_words):
    print(f"read probe: {n_words} words", flush=True)
    g = np.random.default_rng(n_words)
    host = g.integers(0, 2**32, size=n_words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = tidar.read_probe(buf)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("waves_per_simd", [1, 2])
@pytest.mark.parametrize("lds_reads", [False, True])
def test_mfma_probe_records_every_wave(waves_per_simd, lds_reads):
    """The issue-rate probe writes a cycle count for every wave of its
    workgroups, no record carries the impossible-sum mark, and twice the
    rounds take about twice the cycles (the count measures the rounds)."""
    print(f"mfma probe: {waves_per_simd} waves per SIMD, lds {lds_reads}", flush=True)
    short = tidar.mfma_probe(waves_per_simd, lds_reads, 256).cpu().numpy()
    long = tidar.mfma_probe(waves_per_simd, lds_reads, 512).cpu().numpy()
    assert short.shape == (tidar.MFMA_PROBE_BLOCKS * 4 * waves_per_simd,)
    assert (short > 0).all() and (long > 0).all()
    # at least 16 clocks per MFMA (the pipe's own interval) and a round count that scales
    assert np.median(short) >= 16 * 8 * 256
    assert 1.5 < np.median(long) / np.median(short) < 2.5
