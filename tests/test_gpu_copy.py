"""GPU checks of the measurement copies (nrm_bench_copy, nrm_bench_copy2, nrm_bench_copy2_row):
bit-exact copies, including a partial last block and an empty copy."""

import pytest
import torch

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunks", [0, 1, 37, 512, 512 * 3 + 37, 1 << 20])
def test_bench_copies(nrm_lib, chunks):
    say(f"bench copies chunks={chunks}")
    n = 16 * chunks
    g = torch.Generator().manual_seed(chunks)
    s1 = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(DEV)
    s2 = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(DEV)
    d = torch.zeros_like(s1)
    d1, d2 = torch.zeros_like(s1), torch.zeros_like(s1)
    nrm_lib.bench_copy(s1, d)
    nrm_lib.bench_copy2(s1, s2, d1, d2)
    torch.cuda.synchronize()
    assert torch.equal(d, s1)
    assert torch.equal(d1, s1)
    assert torch.equal(d2, s2)


@pytest.mark.parametrize("unit", [8192, 16384, 32768])
@pytest.mark.parametrize("units", [0, 1, 3, 2048])
def test_bench_copy2_row(nrm_lib, unit, units):
    say(f"bench copy2_row unit={unit} units={units}")
    n = unit * units
    g = torch.Generator().manual_seed(units + unit)
    s1 = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(DEV)
    s2 = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(DEV)
    d1, d2 = torch.zeros_like(s1), torch.zeros_like(s1)
    nrm_lib.bench_copy2_row(s1, s2, d1, d2, unit)
    torch.cuda.synchronize()
    assert torch.equal(d1, s1)
    assert torch.equal(d2, s2)
