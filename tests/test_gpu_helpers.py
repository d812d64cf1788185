"""The library's helpers around the linear, on an MI355X: the streaming-read bandwidth
reference (every byte read exactly once: the XOR of the per-workgroup words equals the
XOR of all 32-bit words of the buffer, and a word read twice would cancel) and the
device status word of the fused activation quantization."""
import numpy as np
import pytest
import torch

import bit_weight_quantized_load_amd as qw
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.set_device(0)
    qw.lib()
    yield


@pytest.mark.parametrize("nbytes,waves,blocks,u", [
    (34113536, 0, 0, 0), (67978240, 8, 256, 4), (4096, 1, 1, 1), (1 << 20, 16, 7, 16),
    (16, 4, 3, 2), (1000016, 2, 300, 8)])
def test_stream_read_reads_every_byte_once(nbytes, waves, blocks, u):
    print("stream_read", nbytes, waves, blocks, u, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes % 997)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda",
                        generator=g)
    nb = blocks or torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.full((nb + 8,), 12345, dtype=torch.int32, device="cuda")
    qw.stream_read(src, sink, waves, blocks, u)
    torch.cuda.synchronize()
    s = sink.cpu().numpy().view(np.uint32)
    assert np.all(s[nb:] == 12345)  # nothing written past the workgroups' words
    assert np.bitwise_xor.reduce(s[:nb]) == np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))


def test_device_status_is_clear_after_fused_quantization_runs():
    qw.device_status(clear=True)
    for (N, K) in ((8200, 3584), (512, 3584), (3584, 18944)):
        W = torch.from_numpy(wl.weights(90, 1, N, K)).cuda()
        Wq, s = qw.quantize_pack_w4(W)
        X = torch.from_numpy(wl.activations(90, 2, 1, K)).cuda()
        for _ in range(3):
            qw.gemv_w4a8(X, Wq, s)
        Wg, sg = qw.quantize_pack_w4g(W, 128)
        qw.gemv_w4a8g(X, Wg, sg, N, 128)
    torch.cuda.synchronize()
    assert qw.device_status(clear=True) == 0
