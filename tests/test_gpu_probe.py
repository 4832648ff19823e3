"""The streaming-read probe (a measurement utility of the benchmark, through
the C ABI): every mode reads its buffer and leaves the data it copied in the
sink, including the scattered-page mode over a paged buffer."""
import pytest
import torch

import token_verify_attention_amd as tva
from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("nwg", [1, 256, 1000])
def test_probe_modes_read_the_buffer(mode, nwg):
    say(f"probe mode {mode} workgroups {nwg}")
    nbytes = 64 << 20                                 # 16384 pages of 4 KB
    buf = torch.full((nbytes // 4,), 0x01010101, dtype=torch.int32, device=DEV)
    sink = torch.zeros(nwg * 4, dtype=torch.int32, device=DEV)
    tva.stream_read_probe(buf, mode, nwg, sink)
    torch.cuda.synchronize()
    s = sink.view(nwg, 4).cpu()
    if mode == 0:
        # each wave folds its words by xor: an even or odd count of one word
        assert bool(((s == 0) | (s == 0x01010101)).all())
    else:
        # every wave copied at least one 1 KB block; wave 0 reports its first slot
        assert bool((s[:, 0] == 0x01010101).all())


def test_scattered_pages_need_a_power_of_two():
    buf = torch.zeros(3 * 4096, dtype=torch.uint8, device=DEV)
    with pytest.raises(tva.SvaError, match="power of two"):
        tva.stream_read_probe(buf, 2, 4)
