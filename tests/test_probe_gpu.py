"""The streaming-read probe on the GPU: it reads every byte of its range once.

pbg_stream_read is a measurement helper (the bench times it as the read
ceiling next to the GEMVs), not part of the decode path, so it has no oracle:
its XOR fold, gathered over the sink, must equal numpy's XOR of the range's
32-bit words, which no skipped or repeated chunk can keep.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pbg(gpu):
    import packed_bit_gemv_amd as m

    m.lib()
    return m


def fold(sink) -> int:
    return int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))


# below 8 MiB (one load per lane): one chunk, one workgroup less a chunk /
# exactly / plus a chunk, a ragged multi-workgroup size; from 8 MiB (four loads
# per lane): its first size, a ragged one and the 12288 x 4096 packed matrix;
# from 16 MiB (512 threads): its first size and a ragged 25 MB range
@pytest.mark.parametrize("nbytes", [16, 16 * 255, 16 * 256, 16 * 257, 16 * 300_001, 8 << 20, (8 << 20) + 16 * 1025,
                                    12_582_912, 16 << 20, 25_165_840])
def test_stream_read_folds_every_word(pbg, nbytes):
    say(f"stream_read bytes={nbytes}")
    words = np.random.default_rng(20261203 + nbytes).integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64)
    words = words.astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = pbg.stream_read(src)
    torch.cuda.synchronize()
    assert fold(sink) == int(np.bitwise_xor.reduce(words))
    # a second read of the same range cancels the first
    pbg.stream_read(src, sink)
    torch.cuda.synchronize()
    assert fold(sink) == 0


def test_stream_read_offset_view(pbg):
    say("stream_read offset view")
    words = np.random.default_rng(7).integers(0, 2 ** 32, 4096, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = pbg.stream_read(src[4:4 + 2048])   # 16 bytes in: still 16-byte aligned
    torch.cuda.synchronize()
    assert fold(sink) == int(np.bitwise_xor.reduce(words[4:4 + 2048]))


def test_stream_read_rejects_bad_ranges(pbg):
    say("stream_read bad ranges")
    src = torch.zeros(1024, dtype=torch.int32, device="cuda:0")
    with pytest.raises(pbg.PbgError):
        pbg.stream_read(src[1:5])            # 4-byte offset: misaligned
    with pytest.raises(pbg.PbgError):
        pbg.stream_read(src[:3])             # 12 bytes: not a whole chunk
    torch.cuda.synchronize()
