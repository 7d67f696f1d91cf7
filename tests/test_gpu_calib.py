"""GPU check of the streaming-read probe used for the bandwidth calibration:
it must read every byte of the buffer once (the XOR of its per-block sink
equals the XOR of every 32-bit word of the buffer), including a size below
one block's 64 KiB chunk, sizes with a partial last chunk, and more blocks
than the sink has words."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 20) + 48, (2049 << 16) + 4096 * 16 + 16])
def test_stream_read_reads_every_word(nbytes):
    import sparse_expert_gemv_amd as sg
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[gpu-case] calib stream read of {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda")
    sink = torch.zeros(sg.CALIB_SINK_WORDS, dtype=torch.int32, device="cuda")
    sg.calib_stream_read(int(buf.data_ptr()), nbytes, int(sink.data_ptr()),
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_stream_read_rejects_bad_sizes():
    import sparse_expert_gemv_amd as sg
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    buf = torch.zeros(64, dtype=torch.int32, device="cuda")
    sink = torch.zeros(sg.CALIB_SINK_WORDS, dtype=torch.int32, device="cuda")
    for n in (0, 8, 100):
        with pytest.raises(sg.FlintError):
            sg.calib_stream_read(int(buf.data_ptr()), n, int(sink.data_ptr()), None)
