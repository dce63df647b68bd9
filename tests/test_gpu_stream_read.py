"""The streaming-read measurement kernel reads every byte exactly once: each
workgroup's 16-byte XOR checksum equals numpy's over the words that
workgroup owns, for ragged sizes, one or two buffers and several grid sizes."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from fp8_kv_amd import stream_read
    stream_read.load()
    return torch.device("cuda:0")


def expected(words: np.ndarray, blocks: int) -> np.ndarray:
    """Per-workgroup XOR of uint32x4 words: workgroup w owns the contiguous
    words [w*C, (w+1)*C), C = ceil(n / blocks) rounded up to 256."""
    n = words.shape[0]
    c = -(-n // blocks)
    c = -(-c // 256) * 256
    out = np.zeros((blocks, 4), np.uint32)
    for w in range(blocks):
        chunk = words[w * c:(w + 1) * c]
        if chunk.size:
            out[w] = np.bitwise_xor.reduce(chunk, axis=0)
    return out


@pytest.mark.parametrize("nt", [True, False])
@pytest.mark.parametrize("a_words,b_words,blocks", [
    (1, 0, 1), (255, 0, 3), (4096, 4096, 7), (70_001, 12_345, 256), (262_144, 262_144, 2048),
    (3, 5, 64)])
def test_checksums(dev, a_words, b_words, blocks, nt):
    from fp8_kv_amd import stream_read
    print(f"stream_read a={a_words} b={b_words} blocks={blocks} nt={nt}", flush=True)
    rng = np.random.default_rng(a_words + 7 * b_words + blocks)
    a = rng.integers(0, 2**32, size=(a_words, 4), dtype=np.uint32)
    b = rng.integers(0, 2**32, size=(b_words, 4), dtype=np.uint32)
    da = torch.from_numpy(a.view(np.int32)).to(dev)
    db = torch.from_numpy(b.view(np.int32)).to(dev) if b_words else None
    sink = torch.full((blocks, 4), -1, dtype=torch.int32, device=dev)
    stream_read.stream_read(da, db, sink, blocks, nontemporal=nt)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected(np.concatenate([a, b]), blocks))


def test_clock_probe_plausible(dev):
    """The shader-clock probe the benchmark reads after each timed batch
    returns a spin of at least the asked length and a clock between 0.3 and
    4 GHz."""
    from fp8_kv_amd import stream_read

    buf = torch.zeros(2, dtype=torch.int64, device=dev)
    mhz = stream_read.clock_mhz(buf, ticks=1000)
    real = int(buf[0])
    assert real >= 1000
    assert 300.0 < mhz < 4000.0
