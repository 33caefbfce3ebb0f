"""The streaming-read floor kernel (bq_read_floor), the measurement aid the
products' bandwidth is compared against: it must read every byte of the
buffer exactly once, which the XOR of its sink words shows (the XOR of all
32-bit words of the buffer), for sizes below one pass of its grid, with a
ragged last pass, and over many passes."""
import numpy as np
import pytest

from gpu_util import bqmod, log, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 16 * 524288 * 8 + 16 * 777, 64 * 1024 * 1024 + 16 * 5])
def test_floor_reads_every_byte_once(nbytes):
    t, bq = torch(), bqmod()
    log(f"floor nbytes={nbytes}")
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = t.from_numpy(words.view(np.int32)).to("cuda")
    sink = t.full((bq.BQ_FLOOR_SINK_WORDS,), -1, dtype=t.int32, device="cuda")
    bq.bq_read_floor(buf, sink)
    t.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))
