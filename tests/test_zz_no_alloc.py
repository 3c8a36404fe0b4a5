"""vit_forward_static (activations in the library's static device array, no
allocation) against vit_forward (activations in the workspace bound at
vit_create), through the C ABI: bit-identical tokens, taps and descriptors on
two calls in a row, the second with a smaller batch, so that it runs over the
first call's leftover activations at other offsets."""

import ctypes

import numpy as np
import pytest
import torch

import synth
import vision_transformer_encoder_block_amd as vit
from tests.gpu_util import f32_dev, host, require_gpu, say

pytestmark = pytest.mark.gpu

MIB = 1024 * 1024


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_static_forward_matches_workspace_forward():
    cfg = synth.preset("vits16_336")          # 446 tokens, the 2.3e6-logit sink in block 1
    P = synth.make_params(cfg)
    enc = vit.Encoder(cfg, P, max_batch=8)
    bare = vit.Encoder(cfg, P, max_batch=8, workspace=False)
    for batch, seed in ((8, 31), (3, 32)):
        say(f"static forward, ViT-S/16 @336 batch {batch}")
        x = f32_dev(synth.make_images(cfg, batch, seed=seed))
        t_ws = enc.forward(x)
        d_ws = enc.descriptor(t_ws)
        t_st = enc.forward_static(x)
        d_st = enc.descriptor(t_st)
        t_bare = bare.forward_static(x)
        a, b, c = host(t_ws), host(t_st), host(t_bare)
        assert np.isfinite(a).all()
        np.testing.assert_array_equal(b, a)
        np.testing.assert_array_equal(c, a)
        np.testing.assert_array_equal(host(d_st), host(d_ws))
    enc.close()
    bare.close()


def test_static_forward_with_taps_and_a_smaller_second_call():
    cfg = synth.preset("vits14_518")          # 1370 tokens, taps after blocks 3/6/9/12
    P = synth.make_params(cfg)
    enc = vit.Encoder(cfg, P, max_batch=4)
    for batch, seed in ((4, 41), (1, 42)):
        say(f"static forward with taps, DINOv2-S/14 @518 batch {batch}")
        x = f32_dev(synth.make_images(cfg, batch, seed=seed))
        t_ws, p_ws = enc.forward(x, with_taps=True)
        t_st, p_st = enc.forward_static(x, with_taps=True)
        np.testing.assert_array_equal(host(t_st), host(t_ws))
        np.testing.assert_array_equal(host(p_st), host(p_ws))
    enc.close()


def test_static_forward_size_limit_and_refusals():
    """ViT-L/16 @1024 at batch 1 (94.2 MiB of activations) fits the 96 MiB
    array; batch 2 is refused before anything is enqueued, and so are calls on
    a model without a workspace that need one."""
    cfg = synth.preset("vitl16_1024")
    P = synth.make_params(cfg)
    enc = vit.Encoder(cfg, P, max_batch=2)
    L = vit.lib()
    x = f32_dev(synth.make_images(cfg, 2, seed=51))
    say("static forward, ViT-L/16 @1024 batch 1")
    t_ws = enc.forward(x[:1].contiguous())
    t_st = enc.forward_static(x[:1].contiguous())
    np.testing.assert_array_equal(host(t_st), host(t_ws))
    tok = torch.empty((2, enc.tokens, cfg["dim"]), dtype=torch.float32, device="cuda")
    stream = vit._stream(None)
    assert L.vit_forward_static(enc.handle, x.data_ptr(), 2, tok.data_ptr(), None, stream) == -3
    assert "static scratch holds" in vit.vit_last_error()
    assert L.vit_forward_static(enc.handle, x.data_ptr(), 3, tok.data_ptr(), None, stream) == -3   # > max_batch
    assert L.vit_forward_static(None, x.data_ptr(), 1, tok.data_ptr(), None, stream) == -1
    assert L.vit_forward_static(enc.handle, x.data_ptr(), 1, tok.data_ptr() + 4, None, stream) == -1
    torch.cuda.synchronize()
    enc.close()
    small = synth.preset("vits16_224", img_h=48, img_w=32, dim=128, heads=2, mlp_hidden=256, depth=1,
                         bf16_params=True)
    bare = vit.Encoder(small, synth.make_params(small), max_batch=1, workspace=False)
    xs = f32_dev(synth.make_images(small, 1))
    ts = torch.empty((1, bare.tokens, 128), dtype=torch.float32, device="cuda")
    assert L.vit_forward(bare.handle, xs.data_ptr(), 1, ts.data_ptr(), None, stream) == -1
    assert "workspace" in vit.vit_last_error()
    assert L.vit_forward_static(bare.handle, xs.data_ptr(), 1, ts.data_ptr(), None, stream) == 0
    torch.cuda.synchronize()
    assert np.isfinite(host(ts)).all()
    bare.close()
