"""Decode steps captured in a HIP graph replay to the eager results: several
replays, with eager library work and synchronisations between them, each
checked bitwise against the eager run (same kernels, same inputs)."""
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


def test_decode_graph_replays_match_eager():
    note("graph replay of 24 decode steps, ratio 4, batch 8, dim 256")
    rng = np.random.default_rng(3)
    ratio, hd, dim, batch, steps = 4, 128, 256, 8, 24
    cfg = kvc.Config(ratio, hd, dim)
    proj = kvc.kvc_proj_width(cfg)
    d = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    x = d(rng.standard_normal((steps, batch, dim), dtype=np.float32))
    w = kvc.Weights(d(rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.05)),
                    d(rng.standard_normal((proj, dim), dtype=np.float32) * np.float32(0.05)),
                    d(rng.standard_normal((ratio, proj), dtype=np.float32) * np.float32(0.1)))
    ws = kvc.new_decode_workspace(cfg, batch)
    state = kvc.new_state(cfg, batch)
    groups = steps // ratio
    lat = torch.zeros((groups, batch, hd), dtype=torch.bfloat16, device="cuda")
    codes = torch.zeros((groups, batch, hd // 2), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((groups, batch, hd // 16), dtype=torch.uint8, device="cuda")
    outs = [kvc.Outputs(latent=lat[e], codes=codes[e], scales=scales[e]) for e in range(groups)]

    def one_pass():
        e = 0
        for p in range(steps):
            emits = p > 0 and (p + 1) % ratio == 0
            kvc.compressor_decode_step(cfg, w, x[p], batch, p, ws, state[0], state[1], outs[e] if emits else None)
            e += emits

    one_pass()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (lat, codes, scales, state[0], state[1])]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    torch.cuda.synchronize()

    other = torch.empty_like(ws)
    for rep in range(3):
        for t in (lat, codes, scales):
            t.zero_()
        state[0].fill_(7.0)  # the pass from start_pos 0 must rebuild the carry
        state[1].fill_(-3.0)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((lat, codes, scales, state[0], state[1]), ref):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), rep
        # eager library work between replays
        one_pass()
        other.copy_(ws)
        torch.cuda.synchronize()
