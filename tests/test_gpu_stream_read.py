"""GPU check of the streaming-read ceiling kernel (seedlm_stream_read, a
measurement baseline): every 32-bit word of the buffer is read exactly once, so
the XOR of the per-workgroup checksums (the sink starts at zero) equals the XOR
of the buffer's words, bit for bit.  Sizes cover a single 16-byte load (one
workgroup reads, the rest get empty ranges), ranges that do not divide evenly
over the workgroups or the unrolled loop, and a buffer larger than the
last-level cache."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _S():
    import prng_seeded_decode_amd as S

    return S


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, 3 * (1 << 20) + 1024 * 16 * 8 + 32,
                                    300 << 20])
def test_stream_read_checksum_is_exact(nbytes):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S = _S()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(nbytes % 1000003)
    words = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = torch.zeros(S.STREAM_READ_SINK, dtype=torch.int32, device=dev)
    print(f"stream_read {nbytes} bytes", flush=True)
    S.seedlm_stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)


def test_stream_read_rejects_bad_arguments():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S = _S()
    dev = torch.device("cuda:0")
    sink = torch.zeros(S.STREAM_READ_SINK, dtype=torch.int32, device=dev)
    with pytest.raises(S.SeedLMError):
        S.seedlm_stream_read(torch.zeros(6, dtype=torch.int32, device=dev), sink)  # 24 bytes
    with pytest.raises(ValueError):
        S.seedlm_stream_read(torch.zeros(8, dtype=torch.int32, device=dev), sink[:8])
