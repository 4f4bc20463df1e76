"""The allocation-free NVFP4 entry point (nvfp4_quantize_noalloc, static
device scratch) against nvfp4_quantize with a caller workspace: the same
kernels and grids, so every output must be bit-identical, including the
tensor terms.  Two calls in a row per mode, the second on a smaller tensor,
so the second call runs on scratch the first left behind."""
import numpy as np
import pytest
import torch

import microscaling_fp4_quantization_amd as fq

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

MODES = [(fq.FMT_UE4M3, 16, fq.G_DYNAMIC, 0, fq.MSE_REL),
         (fq.FMT_UE4M3, 16, fq.G_GIVEN, 16, fq.MSE_ABS),
         (fq.FMT_UE4M3, 32, fq.G_NONE, 0, fq.MSE_ABS),
         (fq.FMT_UE5M3, 8, fq.G_NONE, 0, fq.MSE_REL),
         (fq.FMT_UE4M3, 16, fq.G_ROW, 16, fq.MSE_ABS)]


def seeded(shape, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
    return torch.from_numpy(a).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("fmt,block,gmode,rotate,kind", MODES)
def test_noalloc_matches_the_workspace_call(fmt, block, gmode, rotate, kind):
    for i, shape in enumerate([(4096, 3584), (67, 768)]):
        print(f"  noalloc fmt={fmt} block={block} gmode={gmode} rot={rotate} shape={shape}", flush=True)
        x = seeded(shape, [114, i, fmt, block, gmode])
        g_in = torch.tensor([3.1e-5], dtype=torch.float32, device=DEV) if gmode == fq.G_GIVEN else None
        a = fq.nvfp4_quantize(x, block, fmt, gmode, g_in, rotate, mse_kind=kind)
        b = fq.nvfp4_quantize_noalloc(x, block, fmt, gmode, g_in, rotate, mse_kind=kind)
        torch.cuda.synchronize()
        assert torch.equal(a.codes, b.codes)
        assert torch.equal(a.scales, b.scales)
        assert torch.equal(a.block_mse.view(torch.int32), b.block_mse.view(torch.int32))
        assert torch.equal(a.stats.view(torch.int64), b.stats.view(torch.int64))
        if a.g is not None:
            assert torch.equal(a.g.view(torch.int32), b.g.view(torch.int32))
