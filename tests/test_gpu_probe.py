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


@pytest.mark.parametrize("units,read_bytes,write_bytes", [(37, 16384, 10240), (5, 4096, 16), (3, 32768, 65536),
                                                          (9, 8192, 0)])
def test_rw_probe_writes_the_documented_words(units, read_bytes, write_bytes):
    require_gpu()
    rng = np.random.default_rng(units + read_bytes)
    words = rng.integers(0, 2**32, size=(units, read_bytes // 16, 4), dtype=np.uint32)
    src = torch.from_numpy(words.reshape(-1).view(np.uint8).copy()).cuda()
    guard = 256
    dst = torch.full((units * write_bytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    kvq.rw_probe(src, dst[:max(units * write_bytes, 16)], read_bytes, write_bytes)   # 16: a real pointer
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    assert np.all(got[units * write_bytes:] == 0xA5)                      # nothing past the output
    got = got[:units * write_bytes].view(np.uint32).reshape(units, write_bytes // 16, 4)
    # thread t of unit u folds the unit's words t, t + 256, ... and writes w + j to words j = t, t + 256, ...
    for u in range(units):
        fold = np.bitwise_xor.reduce(words[u].reshape(-1, 256, 4), axis=0)   # [thread][lane]
        for j in range(write_bytes // 16):
            assert np.array_equal(got[u, j], fold[j % 256] + np.uint32(j)), (u, j)
