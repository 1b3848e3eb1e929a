"""GPU checks of dflash_hbm_ceiling, the measurement stream the benchmark
reads the kernels against: the copy moves every byte (sizes that end inside
a wave's piece and inside the grid), the read runs and leaves its sink alone
unless the data holds its one bit pattern."""
import pytest
import torch

import block_draft_proposal_amd as D
from gpu_helpers import DEV, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 1008, 1024 * 16 * 4 + 48, (1 << 24) + 16 * 77])
def test_copy_moves_every_byte(nbytes):
    require_gpu()
    say(f"hbm_ceiling copy {nbytes} bytes")
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to(DEV)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    D.dflash_hbm_ceiling(D.CEILING_COPY, src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert int(dst[nbytes:].sum()) == 0          # nothing past the end


def test_read_leaves_the_sink_alone():
    require_gpu()
    say("hbm_ceiling read 64 MiB")
    src = torch.zeros(1 << 24, dtype=torch.int32, device=DEV)   # XOR of zeros never matches the pattern
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    D.dflash_hbm_ceiling(D.CEILING_READ, src, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 7
