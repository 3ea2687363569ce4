"""kvq_stream_read (the read-only bandwidth reference of the measurements) on
the GPU: it reads every 16-byte chunk of the buffer, first and last included,
at sizes that do not fill its slices evenly. Each lane folds its chunks into an
XOR and stores it to the sink only when the fold equals 0x9E3779B9, so a buffer
of zeros with that word in one chunk makes exactly the lane that read it write
the sink; an all-zero buffer leaves the sink alone."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9
SENTINEL = 0x12345678


def _read(buf_words, n_cu):
    import int8_quantized_kv_quant_amd as kvq
    buf = torch.from_numpy(buf_words.view(np.int32)).cuda()
    sink = torch.tensor([SENTINEL], dtype=torch.int32, device="cuda")
    kvq.kvq_stream_read(buf, buf.numel() * 4, sink, n_cu)
    torch.cuda.synchronize()
    return int(sink.cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("n_chunks", [1, 255, 4097, 65536 + 7, (1 << 20) + 3])
@pytest.mark.parametrize("n_cu", [1, 256])
def test_every_chunk_is_read(n_chunks, n_cu):
    print(f"[stream] chunks={n_chunks} n_cu={n_cu}", flush=True)
    words = np.zeros(4 * n_chunks, dtype=np.uint32)
    assert _read(words, n_cu) == SENTINEL          # nothing folds to the marker
    for chunk in sorted({0, n_chunks // 2, n_chunks - 1}):
        words[:] = 0
        words[4 * chunk + (chunk % 4)] = MAGIC
        assert _read(words, n_cu) == MAGIC, chunk   # the lane holding that chunk saw it
