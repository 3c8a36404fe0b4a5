"""Host-side checks of libvit (no GPU needed): the library loads and exports every
function the headers declare, the presets match the workload table, vit_plan's
geometry and sizes, argument validation, and the parameter blob packing."""

import ctypes
import os
import re

import numpy as np
import pytest

import synth
import vision_transformer_encoder_block_amd as vit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vit.LIB_PATH):
        from vision_transformer_encoder_block_amd import build
        build.build(verbose=False)
    return vit.lib()


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(vit_\w+)\s*\(", text, flags=re.M)
    return names


def test_library_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 12
    lib = ctypes.CDLL(vit.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(vit._SIGNATURES)


PRESET_NAMES = ["vits16_224", "vits16_336", "vits14_518", "vitl16_1024", "vitl16_text"]


@pytest.mark.parametrize("cid,name", list(enumerate(PRESET_NAMES, 1)))
def test_presets_match_workloads(L, cid, name):
    c = vit.vit_config_preset(cid)
    ref = vit.config_from_dict(synth.preset(name))
    assert c.as_dict() == pytest.approx(ref.as_dict())
    s = vit.vit_plan(c)
    cfg = synth.preset(name)
    assert s.tokens == synth.tokens(cfg)
    P = synth.make_params(dict(cfg, depth=1, extra_blocks=0)) if cid in (4, 5) else synth.make_params(cfg)
    if cid not in (4, 5):
        assert s.host_floats == vit.pack_params(P).size
    assert s.taps == len(cfg["taps"])


def test_plan_token_counts_and_windows(L):
    s = vit.vit_plan(vit.vit_config_preset(2))
    assert s.tokens == 446
    s = vit.vit_plan(vit.vit_config_preset(3))
    assert s.tokens == 1370 and s.taps == 4
    s = vit.vit_plan(vit.vit_config_preset(4))
    assert s.tokens == 4101
    s = vit.vit_plan(vit.vit_config_preset(5))
    assert s.tokens == 2053 and s.window_tokens == 581 and s.windows == 10


def test_blob_size_matches_pack(L):
    cfg = synth.preset("vits16_224", depth=2, img_h=48, img_w=32, dim=128, heads=2, mlp_hidden=512)
    P = synth.make_params(cfg)
    s = vit.vit_plan(vit.config_from_dict(cfg))
    assert s.host_floats == vit.pack_params(P).size


def _code(fn, *args):
    return fn(*args)


def test_plan_rejects_bad_configs(L):
    lib = L
    out = vit.VitSizes()
    base = vit.vit_config_preset(2)

    def plan(**kw):
        c = vit.VitConfig(**{**base.as_dict(), **kw})
        return lib.vit_plan(ctypes.byref(c), ctypes.byref(out))

    assert plan() == 0
    assert plan(img_h=337) == -2          # not a multiple of the patch
    assert plan(heads=5) == -5            # heads * 64 != dim
    assert plan(dim=1088, heads=17) == -5  # unsupported width
    assert plan(mlp_hidden=1500) == -5
    assert plan(max_batch=0) == -1
    assert plan(ln_eps=0.0) == -1
    assert plan(tap_mask=1 << 12) == -1   # block 13 of 12
    assert plan(window=100, window_stride=50) == -2
    assert "multiple" in vit.vit_last_error()
    # a stride past the window would leave pixels that no window covers
    base5 = vit.vit_config_preset(5).as_dict()
    c5 = vit.VitConfig(**{**base5, "window_stride": 500})
    assert lib.vit_plan(ctypes.byref(c5), ctypes.byref(out)) == -2
    assert "window_stride" in vit.vit_last_error()
    c5 = vit.VitConfig(**{**base5, "window_stride": 384})
    assert lib.vit_plan(ctypes.byref(c5), ctypes.byref(out)) == 0
    assert lib.vit_plan(None, ctypes.byref(out)) == -1
    assert lib.vit_config_preset(9, ctypes.byref(vit.VitConfig())) == -1


def test_create_and_calls_validate_before_touching_the_device(L):
    lib = L
    c = vit.vit_config_preset(1)
    h = ctypes.c_void_p()
    # NULL blob / buffers: rejected on the host
    assert lib.vit_create(ctypes.byref(c), None, 0, None, 0, None, 0, None, ctypes.byref(h)) == -1
    s = vit.vit_plan(c)
    blob = np.zeros(s.host_floats - 1, dtype=np.float32)
    fake = ctypes.c_void_p(0x1000)
    assert lib.vit_create(ctypes.byref(c), blob.ctypes.data_as(ctypes.c_void_p), blob.size, fake, s.weight_bytes,
                          fake, s.workspace_bytes, None, ctypes.byref(h)) == -3
    blob = np.zeros(s.host_floats, dtype=np.float32)
    assert lib.vit_create(ctypes.byref(c), blob.ctypes.data_as(ctypes.c_void_p), blob.size, fake,
                          s.weight_bytes - 1, fake, s.workspace_bytes, None, ctypes.byref(h)) == -3
    assert lib.vit_forward(None, fake, 1, fake, None, None) == -1
    assert lib.vit_forward_static(None, fake, 1, fake, None, None) == -1
    assert lib.vit_descriptor(None, fake, 1, fake, None) == -1
    assert lib.vit_patch_scores(None, fake, fake, 1, 0, fake, None, None, None) == -1
    assert lib.vit_op_linear(fake, fake, fake, 4, 4, 63, 0, None, fake, None) == -2
    assert lib.vit_op_layernorm(fake, 4, 100, fake, fake, ctypes.c_float(1e-6), fake, 0, None) == -2
    assert lib.vit_op_attention(None, fake, fake, 1, 4, 1, fake, None) == -1
    assert lib.vit_op_attention(fake, fake, fake, 0, 4, 1, fake, None) == -2
    f = ctypes.c_float(1e-6)
    assert lib.vit_op_linear_residual_ln(fake, fake, fake, fake, 4, 384, 64, fake, fake, fake, f, None, None) == -1
    assert lib.vit_op_linear_residual_ln(fake, fake, fake, fake, 4, 384, 60, fake, fake, fake, f, fake, None) == -2
    assert lib.vit_op_linear_residual_ln(fake, fake, fake, fake, 4, 512, 64, fake, fake, fake, f, fake, None) == -5
    assert lib.vit_op_preprocess(None, 1, 8, 8, 0, fake, 4, 4, None) == -1
    assert lib.vit_op_preprocess(fake, 1, 8, 8, 0, None, 4, 4, None) == -1
    assert lib.vit_op_preprocess(fake, 0, 8, 8, 0, fake, 4, 4, None) == -2
    assert lib.vit_op_preprocess(fake, 1, 8, 0, 0, fake, 4, 4, None) == -2
    assert lib.vit_op_preprocess(fake, 1, 8, 8, 0, fake, 70000, 4, None) == -2
    assert lib.vit_destroy(None) == 0


# ------------------------------------------------------------------ semantic head (host side)

def test_head_preset_matches_the_diagram(L):
    c = vit.head_config_preset()
    # LibreYOLO DINOv2 diagram: 4 taps of 384 x 37 x 37, projector width 256,
    # GroupNorm 32 groups, 19 classes resized to 518 x 518
    assert (c.grid_h, c.grid_w, c.dim, c.taps, c.width, c.groups, c.classes, c.out_h, c.out_w) == \
        (37, 37, 384, 4, 256, 32, 19, 518, 518)
    assert c.ln_eps == pytest.approx(1e-6) and c.gn_eps == pytest.approx(1e-5)
    s = vit.head_plan(c)
    Ph = synth.make_head_params(synth.preset("vits14_518"))
    assert s.host_floats == vit.pack_head_params(Ph).size
    assert s.weight_bytes > 2 * s.host_floats // 2 and s.workspace_bytes > 0


def test_head_plan_rejects_bad_configs(L):
    lib = ctypes.CDLL(vit.LIB_PATH)

    def plan(**kw):
        c = vit.head_config_preset()
        for k, v in kw.items():
            setattr(c, k, v)
        out = vit.HeadSizes()
        return lib.vit_head_plan(ctypes.byref(c), ctypes.byref(out))

    assert plan() == 0
    assert plan(width=128, groups=16) == -5     # the diagram's width 256 only
    assert plan(width=192, groups=24) == -5
    assert plan(groups=16) == -5                 # width must be 8 * groups
    assert plan(dim=100) == -5
    assert plan(classes=0) == -1
    assert plan(max_batch=0) == -1
    assert plan(grid_h=0) == -2
    assert plan(ln_eps=0.0) == -1
    assert lib.vit_head_plan(None, ctypes.byref(vit.HeadSizes())) == -1


def test_head_create_validates_before_touching_the_device(L):
    lib = ctypes.CDLL(vit.LIB_PATH)
    c = vit.head_config_preset()
    s = vit.head_plan(c)
    blob = np.zeros(s.host_floats - 1, np.float32)
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(256)
    r = lib.vit_head_create(ctypes.byref(c), blob.ctypes.data_as(ctypes.c_void_p), ctypes.c_size_t(blob.size), fake,
                            ctypes.c_size_t(s.weight_bytes), fake, ctypes.c_size_t(s.workspace_bytes), None,
                            ctypes.byref(h))
    assert r == -3 and not h.value
    assert b"floats" in vit.lib().vit_last_error()
    assert lib.vit_head_forward(None, None, 1, None, None, None) == -1
