"""compressor_decode_step_noalloc (no workspace: the library's own scratch
array) against compressor_decode_step on the same inputs, bit for bit:
streams of steps at batch 64, at 256 (the largest batch the scratch holds at
this width) and at 17 (the scratch's arrival counters must be back at zero
and its partial sums are laid out anew), from f32 and from bf16 hidden
states."""
import numpy as np
import pytest
import torch

import kv_cache_compression_fp32_amd.kvc as kvc
from gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvc.lib()


def _host(out):
    return [t.view(torch.uint8).cpu().numpy() if t.dtype != torch.uint8 else t.cpu().numpy()
            for t in (out.latent, out.pooled, out.codes, out.scales, out.dequant)]


@pytest.mark.parametrize("x_format", [kvc.KVC_X_F32, kvc.KVC_X_BF16])
def test_noalloc_decode_matches_the_workspace_decode(x_format):
    rng = np.random.default_rng(23 + x_format)
    cfg = kvc.Config(4, 512, 1024, x_format=x_format)
    proj = kvc.kvc_proj_width(cfg)
    d = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    w = kvc.Weights(d(rng.standard_normal((proj, 1024), dtype=np.float32) * np.float32(0.03)),
                    d(rng.standard_normal((proj, 1024), dtype=np.float32) * np.float32(0.03)),
                    d(rng.standard_normal((4, proj), dtype=np.float32) * np.float32(0.1)))
    # 256 rows at proj 1024 fill the scratch's 2^20 floats of partial sums
    for batch, steps in ((64, 9), (256, 5), (17, 6)):
        note(f"no-alloc decode x_format={x_format} batch={batch} steps={steps}")
        x = d(rng.standard_normal((steps, batch, 1024), dtype=np.float32))
        if x_format == kvc.KVC_X_BF16:
            x = x.to(torch.bfloat16)
        ws = kvc.new_decode_workspace(cfg, batch)
        st_a, st_b = kvc.new_state(cfg, batch), kvc.new_state(cfg, batch)
        emits = 0
        for p in range(steps):
            oa = kvc.new_outputs(cfg, batch, 1, latent=True, pooled=True, fp4=True, dequant=True)
            ob = kvc.new_outputs(cfg, batch, 1, latent=True, pooled=True, fp4=True, dequant=True)
            ea = kvc.compressor_decode_step(cfg, w, x[p], batch, p, ws, st_a[0], st_a[1], oa)
            eb = kvc.compressor_decode_step_noalloc(cfg, w, x[p], batch, p, st_b[0], st_b[1], ob)
            assert ea == eb == (p > 0 and (p + 1) % 4 == 0)
            torch.cuda.synchronize()
            if ea:
                emits += 1
                for a, b in zip(_host(oa), _host(ob)):
                    assert np.array_equal(a, b), p
        assert emits == steps // 4
        assert torch.equal(st_a[0], st_b[0]) and torch.equal(st_a[1], st_b[1])
