"""The C ABI on the CPU: libkvc.so loads, exports every function include/kvc.h
declares, and its host-side logic (sizes, argument checks) answers without
touching a GPU. No call here enqueues work."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import kv_cache_compression_fp32_amd.kvc as kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \t\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("compressor_prefill", "compressor_decode_step", "latent_fp4_quant"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = kvc.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", kvc.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(line.split()[-1] for line in out.stdout.splitlines() if line.strip())
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_strerror():
    assert "gfx950" in kvc.version()
    for code in (0, -1, -2, -3, -4):
        assert kvc.strerror(code)
    assert "unknown" in kvc.strerror(-99)


@pytest.mark.parametrize("ratio,hd,proj,rows", [(2, 512, 512, 2), (4, 512, 1024, 8), (4, 128, 256, 8),
                                                (128, 512, 512, 128), (128, 128, 128, 128)])
def test_sizes(ratio, hd, proj, rows):
    cfg = kvc.Config(ratio, hd, 4096)
    assert kvc.kvc_proj_width(cfg) == proj == cfg.proj
    assert kvc.kvc_state_rows(cfg) == rows == cfg.state_rows
    # the two projection planes and, at ratio 4, the pooled entries of the
    # fused path; by default (f32 x: the f32 matrix cores) then the running
    # sums of a ragged last row tile, 256 rows of both planes' columns
    pooled = 3 * (100 // ratio) * hd if ratio == 4 else 0
    rag = 256 * 2 * proj
    assert kvc.kvc_prefill_workspace_floats(cfg, 3, 100) == 2 * 3 * 100 * proj + pooled + rag
    assert kvc.kvc_prefill_workspace_floats(kvc.Config(ratio, hd, 4096, projection=kvc.KVC_PROJ_F32_MFMA), 3,
                                            100) == 2 * 3 * 100 * proj + pooled + rag
    # the f16 split: two f16 parts [2 proj][2][dim], the exponents of the
    # 2 proj weight rows and of the 300 x rows
    f16_parts = 2 * proj * 4096 + 2 * proj + 300
    cfgh = kvc.Config(ratio, hd, 4096, projection=kvc.KVC_PROJ_F16_SPLIT)
    assert kvc.kvc_prefill_workspace_floats(cfgh, 3, 100) == 2 * 3 * 100 * proj + pooled + f16_parts
    ws = kvc.kvc_decode_workspace_floats(cfg, 64)
    assert ws >= 2 * 2 * 64 * proj and ws % 64 == 0
    # bf16 hidden states (and the bf16 split of f32 x): the weights' three
    # bf16 parts, [2 proj][3][dim]
    parts = 2 * proj * 3 * 4096 // 2
    cfg16 = kvc.Config(ratio, hd, 4096, x_format=kvc.KVC_X_BF16)
    assert kvc.kvc_prefill_workspace_floats(cfg16, 3, 100) == 2 * 3 * 100 * proj + pooled + parts
    assert kvc.kvc_decode_workspace_floats(cfg16, 64) == ws
    cfgb = kvc.Config(ratio, hd, 4096, projection=kvc.KVC_PROJ_BF16_SPLIT)
    assert kvc.kvc_prefill_workspace_floats(cfgb, 3, 100) == 2 * 3 * 100 * proj + pooled + parts


def test_decode_workspace_of_the_b64_ratio4_step():
    # partial sums: from f32 x the two k segments, [2][64][2 x 1024]; from
    # bf16 x the split-K parts (64 column tiles of 32, k split in 4 so that
    # 256 workgroups share the step), [4][2][64][1024]; the larger of the two;
    # then one arrival counter per 32 x 32 tile (2 x 64), rounded up to 64
    cfg = kvc.Config(4, 512, 4096)
    assert kvc.kvc_decode_workspace_floats(cfg, 64) == max(2 * 64 * 2048, 4 * 2 * 64 * 1024) + 128
    # a narrower projection splits bf16 k further, at most 16 ways
    assert kvc.kvc_decode_workspace_floats(kvc.Config(4, 128, 4096), 64) == 16 * 2 * 64 * 256 + 64
    # a ragged batch: 70 rows are 3 tiles of 32 (192 counters); bf16 splits k in 2
    assert kvc.kvc_decode_workspace_floats(cfg, 70) == 2 * 70 * 2048 + 192


@pytest.mark.parametrize("cfg,code", [
    (kvc.Config(3, 512, 4096), kvc.KVC_EUNSUPPORTED),
    (kvc.Config(1, 512, 4096), kvc.KVC_EUNSUPPORTED),
    (kvc.Config(4, 256, 4096), kvc.KVC_EUNSUPPORTED),
    (kvc.Config(4, 512, 4096, eps=-1.0), kvc.KVC_EINVAL),
    (kvc.Config(4, 512, 4096, eps=float("nan")), kvc.KVC_EINVAL),
    (kvc.Config(4, 512, 4096, x_format=2), kvc.KVC_EINVAL),
    (kvc.Config(4, 512, 4096, projection=4), kvc.KVC_EINVAL),
    # the f32 matrix cores and the f16 split read f32 rows only
    (kvc.Config(4, 512, 4096, x_format=kvc.KVC_X_BF16, projection=kvc.KVC_PROJ_F32_MFMA), kvc.KVC_EINVAL),
    (kvc.Config(4, 512, 4096, x_format=kvc.KVC_X_BF16, projection=kvc.KVC_PROJ_F16_SPLIT), kvc.KVC_EINVAL),
])
def test_invalid_configs(cfg, code):
    with pytest.raises(kvc.KvcError) as err:
        kvc.kvc_proj_width(cfg)
    assert err.value.code == code


def _prefill_raw(cfg, **kw):
    lib = kvc.lib()
    args = dict(w=None, x=None, batch=1, seqlen=8, ws=None, ws_n=0, kv=None, sc=None, sb=0, out=None)
    args.update(kw)
    n = ctypes.c_int64(-7)
    w = args["w"]
    rc = lib.compressor_prefill(ctypes.byref(cfg.c()), ctypes.byref(w) if w is not None else None,
                                args["x"], args["batch"], args["seqlen"], args["ws"], args["ws_n"],
                                args["kv"], args["sc"], args["sb"], args["out"], ctypes.byref(n), None)
    return rc, n.value


def test_prefill_argument_errors_return_before_enqueueing():
    cfg = kvc.Config(4, 512, 4096)
    fake = 0x100000  # never dereferenced: every case below fails its host checks
    assert _prefill_raw(kvc.Config(3, 512, 4096))[0] == kvc.KVC_EUNSUPPORTED
    assert _prefill_raw(cfg, batch=0)[0] == kvc.KVC_EINVAL
    assert _prefill_raw(cfg, seqlen=-1)[0] == kvc.KVC_EINVAL
    # projections given (x NULL) but no workspace
    assert _prefill_raw(cfg, seqlen=8)[0] == kvc.KVC_EINVAL
    # workspace too small
    assert _prefill_raw(cfg, seqlen=8, ws=fake, ws_n=10)[0] == kvc.KVC_ESPACE
    # x given without weights
    assert _prefill_raw(cfg, x=fake, ws=fake, ws_n=1 << 30)[0] == kvc.KVC_EINVAL
    # x given with a hidden width that is not a multiple of 32
    w = kvc._Weights(fake, fake, None, None)
    assert _prefill_raw(kvc.Config(4, 512, 100), x=fake, w=w, ws=fake, ws_n=1 << 30)[0] == kvc.KVC_EUNSUPPORTED
    # or one too wide for 32-bit tile offsets
    assert _prefill_raw(kvc.Config(4, 512, (1 << 20) + 32), x=fake, w=w, ws=fake,
                        ws_n=1 << 40)[0] == kvc.KVC_EUNSUPPORTED
    # misaligned pointer
    assert _prefill_raw(cfg, x=fake + 4, w=w, ws=fake, ws_n=1 << 30)[0] == kvc.KVC_EINVAL
    # one state plane without the other, or a state smaller than the batch
    assert _prefill_raw(cfg, ws=fake, ws_n=1 << 30, kv=fake)[0] == kvc.KVC_EINVAL
    assert _prefill_raw(cfg, batch=2, ws=fake, ws_n=1 << 30, kv=fake, sc=fake, sb=1)[0] == kvc.KVC_EINVAL


@pytest.mark.parametrize("x_format", [kvc.KVC_X_F32, kvc.KVC_X_BF16])
def test_projection_needs_room_for_the_split_weights(x_format):
    fake = 0x100000  # never dereferenced: every case below fails its host checks
    w = kvc._Weights(fake, fake, None, None)
    cfg = kvc.Config(4, 512, 4096, x_format=x_format, projection=kvc.KVC_PROJ_BF16_SPLIT)
    full = kvc.kvc_prefill_workspace_floats(cfg, 1, 8)
    planes = 2 * 8 * 1024 + 2 * 512   # the projection planes and the pooled rows
    assert full == planes + 2 * 1024 * 3 * 4096 // 2
    # with x the three-part weights must fit after them
    assert _prefill_raw(cfg, x=fake, w=w, ws=fake, ws_n=planes)[0] == kvc.KVC_ESPACE
    assert _prefill_raw(cfg, x=fake, w=w, ws=fake, ws_n=full - 1)[0] == kvc.KVC_ESPACE
    # without x only the planes are read
    assert _prefill_raw(cfg, ws=fake, ws_n=10)[0] == kvc.KVC_ESPACE
    # x must be 16-byte aligned
    assert _prefill_raw(cfg, x=fake + 2, w=w, ws=fake, ws_n=full)[0] == kvc.KVC_EINVAL


def test_f16_split_projection_needs_room_for_parts_and_exponents():
    fake = 0x100000  # never dereferenced: every case below fails its host checks
    w = kvc._Weights(fake, fake, None, None)
    cfg = kvc.Config(4, 512, 4096, projection=kvc.KVC_PROJ_F16_SPLIT)
    full = kvc.kvc_prefill_workspace_floats(cfg, 1, 8)
    planes = 2 * 8 * 1024 + 2 * 512
    assert full == planes + 2 * 1024 * 4096 + 2 * 1024 + 8
    assert _prefill_raw(cfg, x=fake, w=w, ws=fake, ws_n=full - 1)[0] == kvc.KVC_ESPACE
    assert _prefill_raw(cfg, x=fake, w=w, ws=fake, ws_n=planes + 2 * 1024 * 4096)[0] == kvc.KVC_ESPACE


def test_f32_matrix_core_projection_needs_the_planes_and_the_ragged_tile_sums():
    fake = 0x100000
    w = kvc._Weights(fake, fake, None, None)
    cfg = kvc.Config(4, 512, 4096, projection=kvc.KVC_PROJ_F32_MFMA)
    full = kvc.kvc_prefill_workspace_floats(cfg, 1, 8)
    assert full == 2 * 8 * 1024 + 2 * 512 + 256 * 2048
    assert _prefill_raw(cfg, x=fake, w=w, ws=fake, ws_n=full - 1)[0] == kvc.KVC_ESPACE
    # without x only the planes are read
    assert _prefill_raw(cfg, ws=fake, ws_n=2 * 8 * 1024 - 1)[0] == kvc.KVC_ESPACE


def test_decode_argument_errors_return_before_enqueueing():
    lib = kvc.lib()
    cfg = kvc.Config(4, 512, 4096)
    fake = 0x100000
    e = ctypes.c_int32(-1)

    def call(**kw):
        a = dict(x=None, batch=1, pos=5, ws=fake, ws_n=1 << 30, kv=fake, sc=fake, sb=1)
        a.update(kw)
        return lib.compressor_decode_step(ctypes.byref(cfg.c()), None, a["x"], a["batch"], a["pos"], a["ws"],
                                          a["ws_n"], a["kv"], a["sc"], a["sb"], None, ctypes.byref(e), None)
    assert call(pos=-1) == kvc.KVC_EINVAL
    assert call(kv=None) == kvc.KVC_EINVAL
    assert call(ws=None) == kvc.KVC_EINVAL
    assert call(ws_n=2 * 1024 - 1) == kvc.KVC_ESPACE
    # the partial sums fit but the arrival counters after them do not
    assert call(ws_n=kvc.kvc_decode_workspace_floats(cfg, 1) - 1) == kvc.KVC_ESPACE
    assert call(batch=2, sb=1) == kvc.KVC_EINVAL


def test_fp4_argument_errors():
    lib = kvc.lib()
    fake = 0x100000
    assert lib.latent_fp4_quant(fake, 4, 24, None, None, None, None) == kvc.KVC_EINVAL   # width % 16
    assert lib.latent_fp4_quant(fake, -1, 32, None, None, None, None) == kvc.KVC_EINVAL
    assert lib.latent_fp4_quant(None, 4, 32, None, None, None, None) == kvc.KVC_EINVAL
    # partially overlapping input and output
    assert lib.latent_fp4_quant(fake, 4, 32, None, None, fake + 64, None) == kvc.KVC_EINVAL
    # nothing to do: no launch
    assert lib.latent_fp4_quant(None, 0, 32, None, None, None, None) == kvc.KVC_OK
    # the indexer's form works on blocks of 32
    assert lib.indexer_fp4_quant(fake, 4, 48, None, None, None, None) == kvc.KVC_EINVAL
    assert lib.indexer_fp4_quant(None, 0, 64, None, None, None, None) == kvc.KVC_OK


def test_fp4_format_is_checked():
    with pytest.raises(kvc.KvcError):
        kvc.kvc_proj_width(kvc.Config(4, 512, 4096, fp4_format=7))
    assert kvc.kvc_proj_width(kvc.Config(4, 512, 4096, fp4_format=kvc.KVC_FP4_E8M0_B32)) == 1024


def test_ratio1_argument_errors_return_before_enqueueing():
    lib = kvc.lib()
    fake = 0x100000

    def call(cfg, **kw):
        a = dict(wkv=fake, norm=None, x=fake, tokens=8, ws=fake, ws_n=1 << 30, out=None)
        a.update(kw)
        return lib.compressor_ratio1_forward(ctypes.byref(cfg.c()), a["wkv"], a["norm"], a["x"], a["tokens"],
                                             a["ws"], a["ws_n"], a["out"], None)
    ok = kvc.Config(1, 512, 4096)
    assert kvc.kvc_ratio1_workspace_floats(ok, 10) == 5120
    with pytest.raises(kvc.KvcError):
        kvc.kvc_ratio1_workspace_floats(kvc.Config(4, 512, 4096), 10)   # the pooled compressor's config
    assert call(kvc.Config(4, 512, 4096)) == kvc.KVC_EINVAL
    assert call(kvc.Config(1, 256, 4096)) == kvc.KVC_EUNSUPPORTED
    assert call(kvc.Config(1, 512, 4096 + 32)) == kvc.KVC_EUNSUPPORTED   # dim % 64
    assert call(kvc.Config(1, 512, 0)) == kvc.KVC_EINVAL
    assert call(ok, tokens=-1) == kvc.KVC_EINVAL
    assert call(ok, x=None) == kvc.KVC_EINVAL
    assert call(ok, wkv=None) == kvc.KVC_EINVAL
    assert call(ok, ws_n=8 * 512 - 1) == kvc.KVC_ESPACE
    assert call(ok, x=fake + 2) == kvc.KVC_EINVAL                          # misaligned
    assert call(ok, tokens=0, x=None, wkv=None, ws=None) == kvc.KVC_OK     # nothing to do
    # and the pooled entry points reject ratio 1
    assert _prefill_raw(kvc.Config(1, 512, 4096))[0] == kvc.KVC_EUNSUPPORTED


def test_rope_arguments_are_checked():
    lib = kvc.lib()
    fake = 0x100000
    # rope_dim: even, within the entry; not offered at ratio 1
    for bad in (3, 514, -2):
        with pytest.raises(kvc.KvcError):
            kvc.kvc_proj_width(kvc.Config(4, 512, 4096, rope_dim=bad))
    assert kvc.kvc_proj_width(kvc.Config(4, 512, 4096, rope_dim=64)) == 1024
    with pytest.raises(kvc.KvcError) as err:
        kvc.kvc_ratio1_workspace_floats(kvc.Config(1, 512, 4096, rope_dim=64), 8)
    assert err.value.code == kvc.KVC_EUNSUPPORTED
    cfg = kvc.Config(4, 512, 4096, rope_dim=64)
    out = kvc._Outputs(fake)  # latent only
    # entries written but no table, or a table with too few rows (16 tokens = 4 entries)
    assert _prefill_raw(cfg, seqlen=16, ws=fake, ws_n=1 << 30, out=ctypes.byref(out))[0] == kvc.KVC_EINVAL
    w = kvc._Weights(None, None, None, None, fake, 3)
    assert _prefill_raw(cfg, w=w, seqlen=16, ws=fake, ws_n=1 << 30, out=ctypes.byref(out))[0] == kvc.KVC_EINVAL
    # a rotated output without RoPE
    rot = kvc._Outputs(None, None, None, None, None, fake)
    assert _prefill_raw(kvc.Config(4, 512, 4096), seqlen=16, ws=fake, ws_n=1 << 30,
                        out=ctypes.byref(rot))[0] == kvc.KVC_EINVAL
    # the standalone rotation
    assert lib.latent_rope(fake, 4, 512, 63, fake, 8, 0, fake, None) == kvc.KVC_EINVAL   # odd rope_dim
    assert lib.latent_rope(fake, 4, 512, 1024, fake, 8, 0, fake, None) == kvc.KVC_EINVAL  # wider than a row
    assert lib.latent_rope(fake, 4, 512, 64, fake, 8, 5, fake, None) == kvc.KVC_EINVAL    # rows past the table
    assert lib.latent_rope(fake, 4, 512, 64, fake + 4, 8, 0, fake, None) == kvc.KVC_EINVAL  # misaligned table
    assert lib.latent_rope(fake, 4, 512, 64, fake, 8, 0, fake + 64, None) == kvc.KVC_EINVAL  # partial overlap
    assert lib.latent_rope(None, 0, 512, 64, None, 0, 0, None, None) == kvc.KVC_OK         # nothing to do


def test_time_hook_arguments():
    lib = kvc.lib()
    fake = 0x100000  # never recorded: the pending request is cleared below
    assert lib.kvc_time_next_projection(fake, None) == kvc.KVC_EINVAL
    assert lib.kvc_time_next_projection(None, fake) == kvc.KVC_EINVAL
    assert lib.kvc_time_next_projection(None, None) == kvc.KVC_OK


# ---------------------------------------------------------------- binding size checks
def _t(shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def _prefill_tensors():
    # ratio 4, head_dim 128 (proj 256, 8 state rows), dim 64, batch 2, 12 tokens (3 entries)
    cfg = kvc.Config(4, 128, 64)
    w = kvc.Weights(_t((256, 64)), _t((256, 64)), _t((4, 256)), _t(128))
    t = dict(x=_t((2, 12, 64)), kv=_t((2, 8, 256)), sc=_t((2, 8, 256)),
             out=kvc.Outputs(latent=_t((2, 3, 128), torch.bfloat16), pooled=_t((2, 3, 128)),
                             codes=_t((2, 3, 64), torch.uint8), scales=_t((2, 3, 8), torch.uint8)))
    return cfg, w, t


@pytest.mark.parametrize("bad,name", [
    ("x", "x"), ("wkv", "wkv"), ("wgate", "wgate"), ("ape", "ape"), ("norm_w", "norm_w"),
    ("kv", "kv_state"), ("sc", "score_state"), ("latent", "latent"), ("pooled", "pooled"),
    ("codes", "codes"), ("scales", "scales"),
])
def test_prefill_binding_rejects_wrong_sizes(bad, name):
    """The C ABI gets bare pointers, so the binding checks every tensor's size
    against the config, batch and seqlen before calling it (no GPU needed:
    the checks come before any device or pointer is looked at)."""
    cfg, w, t = _prefill_tensors()
    if bad in ("wkv", "wgate", "ape", "norm_w"):
        setattr(w, bad, _t(getattr(w, bad).numel() + 4))
    elif bad in ("latent", "pooled", "codes", "scales"):
        o = getattr(t["out"], bad)
        setattr(t["out"], bad, _t((o.shape[0], o.shape[1] + 1, o.shape[2]), o.dtype))
    else:
        o = t[bad]
        t[bad] = _t((o.shape[0], o.shape[1] + 1, o.shape[2]))
    with pytest.raises(ValueError, match=name):
        kvc.compressor_prefill(cfg, w, t["x"], 2, 12, _t(10), t["kv"], t["sc"], t["out"])
    # with every size right, the next check is the device
    cfg, w, t = _prefill_tensors()
    with pytest.raises(ValueError, match="GPU"):
        kvc.compressor_prefill(cfg, w, t["x"], 2, 12, _t(10), t["kv"], t["sc"], t["out"])


def test_state_planes_must_hold_the_batch():
    cfg, w, t = _prefill_tensors()
    with pytest.raises(ValueError, match="batch"):
        kvc.compressor_prefill(cfg, w, t["x"], 3, 8, _t(10), t["kv"], t["sc"])
    with pytest.raises(ValueError, match="together"):
        kvc.compressor_prefill(cfg, w, t["x"], 2, 12, _t(10), t["kv"], None)


def test_decode_binding_rejects_wrong_sizes():
    cfg, w, t = _prefill_tensors()
    one = kvc.Outputs(latent=_t((2, 1, 128), torch.bfloat16))
    with pytest.raises(ValueError, match="x"):
        kvc.compressor_decode_step(cfg, w, _t((2, 65)), 2, 3, _t(10), t["kv"], t["sc"], one)
    with pytest.raises(ValueError, match="latent"):
        kvc.compressor_decode_step(cfg, w, _t((2, 64)), 2, 3, _t(10), t["kv"], t["sc"],
                                   kvc.Outputs(latent=_t((2, 2, 128), torch.bfloat16)))
    with pytest.raises(ValueError, match="state"):
        kvc.compressor_decode_step(cfg, w, _t((2, 64)), 2, 3, _t(10), None, None, one)
    with pytest.raises(ValueError, match="GPU"):
        kvc.compressor_decode_step(cfg, w, _t((2, 64)), 2, 3, _t(10), t["kv"], t["sc"], one)


def test_ratio1_and_quantiser_bindings_reject_wrong_sizes():
    cfg = kvc.Config(1, 128, 64)
    x, wkv = _t((10, 64), torch.bfloat16), _t((128, 64), torch.bfloat16)
    with pytest.raises(ValueError, match="wkv"):
        kvc.compressor_ratio1_forward(cfg, _t((128, 32), torch.bfloat16), x, 10, _t(1280))
    with pytest.raises(ValueError, match="x"):
        kvc.compressor_ratio1_forward(cfg, wkv, x, 11, _t(1280))
    with pytest.raises(ValueError, match="latent"):
        kvc.compressor_ratio1_forward(cfg, wkv, x, 10, _t(1280),
                                      kvc.Outputs(latent=_t((1, 9, 128), torch.bfloat16)))
    inp = _t((4, 64), torch.bfloat16)
    with pytest.raises(ValueError, match="codes"):
        kvc.latent_fp4_quant(inp, codes=_t((4, 31), torch.uint8))
    with pytest.raises(ValueError, match="scales"):
        kvc.latent_fp4_quant(inp, scales=_t((4, 2), torch.uint8))
    with pytest.raises(ValueError, match="scales"):
        kvc.indexer_fp4_quant(inp, scales=_t((4, 4), torch.uint8))   # blocks of 32: 2 per row
    with pytest.raises(ValueError, match="out"):
        kvc.latent_fp4_quant(inp, out=_t((4, 48), torch.bfloat16))
    with pytest.raises(ValueError, match="rope_cs"):
        kvc.latent_rope(inp, 16, _t((4, 16, 2)))


def test_noalloc_decode_limits_are_checked_before_the_gpu():
    """The step without a workspace rejects a missing x and batches whose
    partial sums exceed its 2^20-float scratch before touching a GPU."""
    lib = kvc.lib()
    fake = 0x100000  # never dereferenced: every case below fails its host checks
    e = ctypes.c_int32(-1)

    def call(cfg, x, batch):
        w = kvc._Weights(fake, fake, None, None)
        return lib.compressor_decode_step_noalloc(ctypes.byref(cfg.c()), ctypes.byref(w), x, batch, 3, fake, fake,
                                                  batch, None, ctypes.byref(e), None)
    cfg = kvc.Config(4, 512, 4096)   # proj 1024: 4 * batch * 1024 floats of partial sums
    assert call(cfg, None, 8) == kvc.KVC_EINVAL
    assert call(cfg, fake, 0) == kvc.KVC_EINVAL
    assert call(cfg, fake, 257) == kvc.KVC_ESPACE
    assert call(kvc.Config(4, 128, 4096), fake, 1025) == kvc.KVC_ESPACE   # proj 256
    assert call(kvc.Config(128, 512, 4096), fake, 513) == kvc.KVC_ESPACE  # proj 512
