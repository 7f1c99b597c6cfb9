"""pa_read_probe, the streaming-read measurement helper: every byte of the
buffer is read (the XOR of the per-workgroup words equals the XOR of the
buffer's 32-bit words, computed here with numpy), and bad arguments are
refused before any launch."""

import numpy as np
import pytest
import torch

from gpu_cases import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 16 * 1000 + 16, (4 << 20) + 48, 64 << 20])
def test_every_word_is_read(gpu_lib, nbytes):
    announce("read_probe", nbytes)
    host = np.random.default_rng(nbytes + 5).integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    sink = gpu_lib.pa_read_probe(buf)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) if sink.numel() else 0
    want = np.bitwise_xor.reduce(host.view(np.uint32)) if nbytes else np.uint32(0)
    assert int(got) == int(want)


def test_bad_arguments_are_refused(gpu_lib):
    with pytest.raises(gpu_lib.PagedKVError):
        gpu_lib.pa_read_probe(torch.zeros(17, dtype=torch.uint8, device="cuda"))  # not a multiple of 16
    with pytest.raises(gpu_lib.PagedKVError):
        gpu_lib.pa_read_probe(torch.zeros(64, dtype=torch.uint8, device="cuda")[4:36])  # misaligned
    with pytest.raises(ValueError):
        gpu_lib.pa_read_probe(torch.zeros(64, dtype=torch.uint8, device="cuda"),
                              sink=torch.zeros(16, dtype=torch.int32, device="cuda"))
