"""The GPU twin of the input generator reproduces the numpy generator bit for bit."""
import numpy as np
import pytest
import torch

import workloads
import workloads.gpu as wgen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("sigma", [1.0, 0.5])
def test_gpu_generator_matches_numpy(dtype, sigma):
    for seed, stream, seq, e0, n in [(1, 21, 0, 0, 4096), (3, 22, 255, 12345, 70001), (4, 20, 15, 2 ** 31 + 7, 999),
                                     (2, 21, 51, 5, 1)]:
        key = workloads.hash_key(seed, stream, seq)
        t = torch.empty(n, dtype=dtype, device="cuda")
        wgen.fill(t, key, e0, sigma)
        torch.cuda.synchronize()
        ref = workloads.hash_values(key, e0, e0 + n, sigma)
        if dtype == torch.float32:
            got = t.cpu().numpy()
            assert (got.view(np.uint32) == ref.view(np.uint32)).all()
        else:
            got = t.view(torch.int16).cpu().numpy().view(np.uint16)
            assert (got == workloads.bf16_bits(ref)).all()
