"""GPU check of the diagnostic streaming-read kernel (kvq_read_probe): every 16-byte unit of a
ragged buffer is read exactly once, by the thread the documented partition names."""
import numpy as np
import pytest
import torch

from quantized_kv_cache_quant_amd import kvq

from kvq_testlib import require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,groups", [(3 * 2048 + 777, 3), (5000, 1), (700, 4)])
def test_read_probe_reads_every_unit_once(n16, groups):
    require_gpu()
    rng = np.random.default_rng(7 + n16)
    words = rng.integers(0, 2**32, size=(n16, 4), dtype=np.uint32)
    buf = torch.from_numpy(words.reshape(-1).view(np.uint8).copy()).cuda()
    sink = torch.full((groups * 512,), -1, dtype=torch.int32, device="cuda")
    kvq.read_probe(buf, sink, groups)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    # workgroup g reads units [g * per, min((g + 1) * per, n16)); its thread t the units
    # b + t, b + t + 512, ...; each thread writes the XOR of the words it read
    x = np.bitwise_xor.reduce(words, axis=1)
    per = -(-n16 // groups)
    exp = np.zeros(groups * 512, np.uint32)
    for g in range(groups):
        b, e = g * per, min((g + 1) * per, n16)
        for t in range(512):
            exp[g * 512 + t] = np.bitwise_xor.reduce(x[b + t:e:512]) if b + t < e else 0
    assert np.array_equal(got, exp)
