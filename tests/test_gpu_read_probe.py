"""GPU checks of the streaming-read probe (a measurement aid beside the
attention path): every 16-byte word of the source is read exactly once —
the XOR of the sink words equals the XOR of the source words — including
sizes that do not divide evenly among the probe's workgroups; bad
arguments are rejected before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

pkv = pytest.importorskip("paged_kv_cache_51_amd")

pytestmark = pytest.mark.gpu


def xor_words(a):
    return np.bitwise_xor.reduce(a.view(np.uint32).reshape(-1, 4), axis=0)


@pytest.mark.parametrize("nbytes", [16, 4096, 3 * (1 << 20) + 48, 64 << 20])
def test_read_probe_reads_every_word_once(nbytes):
    host = np.random.default_rng(nbytes).integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(host).cuda()
    sink = pkv.read_probe(src)
    torch.cuda.synchronize()
    assert np.array_equal(xor_words(sink.cpu().numpy()), xor_words(host))


def test_read_probe_rejects_bad_arguments():
    lib = pkv.lib()
    need = int(lib.pkv_read_probe_sink_bytes())
    assert need > 0 and need % 16 == 0
    src = torch.zeros(64, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ps, pk = ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(sink.data_ptr())
    assert lib.pkv_read_probe(ps, 40, pk, need, None) == -1          # not a multiple of 16
    assert lib.pkv_read_probe(None, 64, pk, need, None) == -1        # null source
    assert lib.pkv_read_probe(ps, 64, pk, need - 16, None) == -2     # sink too small
    assert lib.pkv_read_probe(ps, 0, None, 0, None) == 0             # nothing to read
    torch.cuda.synchronize()
