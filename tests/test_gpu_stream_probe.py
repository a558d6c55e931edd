"""The streaming-read probe behind the bench's measured HBM ceiling
(`pa_stream_read_probe`, a measurement aid, not a step of the method): every
16-byte chunk of the buffer is read exactly once.  Each workgroup folds the
32-bit words of its slab with XOR into one sink word, so the XOR of the sink
equals the XOR of the whole buffer; on random data a chunk skipped or read
twice breaks that equality."""
import numpy as np
import pytest

from tests.gpu_util import announce, need_gpu, torch

pytestmark = pytest.mark.gpu

P = pytest.importorskip("paged_kv_cache_134_amd")


def _xor_all(words: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(words.astype(np.uint32), initial=np.uint32(0)))


@pytest.mark.parametrize("nbytes", [16, 16 * 1001, 4 << 20, (8 << 20) + 48])
def test_probe_reads_every_chunk_once(nbytes):
    need_gpu()
    announce("stream probe", nbytes, "bytes")
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda",
                        generator=g)
    nw = P.pa_stream_read_probe_sink_words()
    sink = torch.full((nw,), -1, dtype=torch.int32, device="cuda")
    P.pa_stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert _xor_all(sink.cpu().numpy()) == _xor_all(buf.cpu().numpy())


def test_probe_rejects_sizes_that_are_not_16_byte_multiples():
    need_gpu()
    buf = torch.zeros(17, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(P.pa_stream_read_probe_sink_words(), dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="multiple of 16"):
        P.pa_stream_read_probe(buf, sink)
