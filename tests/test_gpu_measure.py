"""The benchmark's streaming-read calibration kernel reads every byte: the
XOR of its per-workgroup words equals the XOR of the buffer's 32-bit words
(numpy on the host), for both cache policies and for sizes that end inside
a workgroup's piece."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from paged_kv_cache_261_amd import pa  # noqa: E402


@pytest.mark.parametrize("nbytes", [16, 4096, 32768 + 48, (1 << 27) + 16 * 7, 3 << 28])
@pytest.mark.parametrize("nt", [True, False])
def test_stream_read_reads_every_byte(nbytes, nt):
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(-2**31, 2**31, size=nbytes // 4, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(host).cuda()
    sink = torch.full((pa.MEASURE_SINK_WORDS,), -1, dtype=torch.int32, device="cuda")
    pa.pa_measure_stream_read(buf, sink, nontemporal=nt)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy())
    want = np.bitwise_xor.reduce(host)
    assert got == want
