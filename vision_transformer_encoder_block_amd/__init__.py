"""Python binding of libvit, the MI355X (gfx950) ViT encoder forward pass.

The C ABI (``include/vit.h``, ``include/vit_ops.h``) does all the work; this
module only marshals arguments: it loads ``libvit.so`` with ctypes, mirrors the
C structs, packs a parameter dictionary into the documented fp32 blob order, and
passes torch device pointers and the current HIP stream.  PyTorch supplies the
device memory and the stream; no step of the encoder runs in Python or torch.

Importing this module never touches the GPU.  Calling into the library needs
the built ``libvit.so`` (``python -m vision_transformer_encoder_block_amd.build``)
and raises ``LibraryMissing`` otherwise: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "LibraryMissing", "VitError", "VitConfig", "VitSizes", "lib", "config_from_dict", "pack_params",
    "vit_config_preset", "vit_plan", "vit_create", "vit_forward", "vit_forward_static", "vit_descriptor", "vit_patch_scores",
    "vit_destroy", "vit_last_error", "vit_op_layernorm", "vit_op_linear", "vit_op_qkv", "vit_op_attention",
    "vit_op_preprocess", "vit_op_linear_residual_ln",
    "Encoder", "EncoderGraph", "EPI_BIAS_BF16", "EPI_GELU_BF16", "EPI_RESIDUAL", "EPI_BIAS_F32",
    "HeadConfig", "HeadSizes", "head_config_preset", "head_config", "head_plan", "pack_head_params", "SemanticHead",
    "vit_op_conv3x3", "vit_op_convx", "vit_op_absmax", "vit_op_quantize_fp8", "vit_op_linear_fp8",
    "vit_op_quantize_int8", "vit_op_linear_int8",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvit.so")

EPI_BIAS_BF16, EPI_GELU_BF16, EPI_RESIDUAL, EPI_BIAS_F32 = 0, 1, 2, 3
STATUS = {0: "VIT_OK", -1: "VIT_ERR_ARG", -2: "VIT_ERR_SHAPE", -3: "VIT_ERR_SIZE", -4: "VIT_ERR_HIP",
          -5: "VIT_ERR_UNSUPPORTED"}


class LibraryMissing(RuntimeError):
    pass


class VitError(RuntimeError):
    def __init__(self, func, code, msg):
        super().__init__(f"{func} -> {STATUS.get(code, code)}: {msg}")
        self.code = code


class VitConfig(ctypes.Structure):
    _fields_ = [
        ("img_h", ctypes.c_int), ("img_w", ctypes.c_int), ("patch", ctypes.c_int), ("dim", ctypes.c_int),
        ("depth", ctypes.c_int), ("extra_blocks", ctypes.c_int), ("heads", ctypes.c_int),
        ("mlp_hidden", ctypes.c_int), ("registers", ctypes.c_int), ("max_batch", ctypes.c_int),
        ("ln_eps", ctypes.c_float), ("tap_mask", ctypes.c_uint), ("pos_grid_h", ctypes.c_int),
        ("pos_grid_w", ctypes.c_int), ("window", ctypes.c_int), ("window_stride", ctypes.c_int),
        ("max_classes", ctypes.c_int),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class VitSizes(ctypes.Structure):
    _fields_ = [
        ("weight_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t), ("host_floats", ctypes.c_size_t),
        ("tokens", ctypes.c_int), ("window_tokens", ctypes.c_int), ("windows", ctypes.c_int), ("taps", ctypes.c_int),
    ]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int

_SIGNATURES = {
    "vit_last_error": (ctypes.c_char_p, []),
    "vit_config_preset": (_I, [_I, ctypes.POINTER(VitConfig)]),
    "vit_plan": (_I, [ctypes.POINTER(VitConfig), ctypes.POINTER(VitSizes)]),
    "vit_create": (_I, [ctypes.POINTER(VitConfig), _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P,
                        ctypes.POINTER(_P)]),
    "vit_forward": (_I, [_P, _P, _I, _P, _P, _P]),
    "vit_forward_static": (_I, [_P, _P, _I, _P, _P, _P]),
    "vit_descriptor": (_I, [_P, _P, _I, _P, _P]),
    "vit_patch_scores": (_I, [_P, _P, _P, _I, _I, _P, _P, _P, _P]),
    "vit_destroy": (_I, [_P]),
    "vit_op_layernorm": (_I, [_P, _I, _I, _P, _P, ctypes.c_float, _P, _I, _P]),
    "vit_op_linear": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "vit_op_qkv": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P]),
    "vit_op_attention": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "vit_op_preprocess": (_I, [_P, _I, _I, _I, _I, _P, _I, _I, _P]),
    "vit_op_linear_residual_ln": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _P, _P, ctypes.c_float, _P, _P]),
    "vit_head_config_preset": (_I, [_P]),
    "vit_head_plan": (_I, [_P, _P]),
    "vit_head_create": (_I, [_P, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P, ctypes.c_size_t, _P,
                             ctypes.POINTER(_P)]),
    "vit_head_forward": (_I, [_P, _P, _I, _P, _P, _P]),
    "vit_head_destroy": (_I, [_P]),
    "vit_op_conv3x3": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P]),
    "vit_op_convx": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, ctypes.c_float, _P, _I, _I, _P]),
    "vit_op_absmax": (_I, [_P, _I, ctypes.c_size_t, _P, _P]),
    "vit_op_quantize_fp8": (_I, [_P, _I, ctypes.c_size_t, ctypes.c_float, _P, _P]),
    "vit_op_linear_fp8": (_I, [_P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _I, _P]),
    "vit_op_quantize_int8": (_I, [_P, _I, ctypes.c_size_t, ctypes.c_float, _P, _P]),
    "vit_op_linear_int8": (_I, [_P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _I, _P]),
}


def lib():
    """The loaded libvit (raises LibraryMissing if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(f"{LIB_PATH} not built; run python -m vision_transformer_encoder_block_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def vit_last_error() -> str:
    return lib().vit_last_error().decode()


def _check(name, code):
    if code != 0:
        raise VitError(name, code, vit_last_error())
    return code


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ C ABI, same names

def vit_config_preset(cfg_id: int) -> VitConfig:
    c = VitConfig()
    _check("vit_config_preset", lib().vit_config_preset(cfg_id, ctypes.byref(c)))
    return c


def vit_plan(cfg: VitConfig) -> VitSizes:
    s = VitSizes()
    _check("vit_plan", lib().vit_plan(ctypes.byref(cfg), ctypes.byref(s)))
    return s


def vit_create(cfg: VitConfig, blob: np.ndarray, d_weights, d_workspace, stream=None):
    blob = np.ascontiguousarray(blob, dtype=np.float32)
    handle = ctypes.c_void_p()
    _check("vit_create", lib().vit_create(
        ctypes.byref(cfg), blob.ctypes.data_as(ctypes.c_void_p), blob.size, _ptr(d_weights),
        d_weights.numel() * d_weights.element_size(), _ptr(d_workspace),
        0 if d_workspace is None else d_workspace.numel() * d_workspace.element_size(), _stream(stream),
        ctypes.byref(handle)))
    return handle


def vit_forward(handle, d_images, batch, d_tokens, d_taps=None, stream=None):
    return _check("vit_forward", lib().vit_forward(handle, _ptr(d_images), batch, _ptr(d_tokens), _ptr(d_taps),
                                                   _stream(stream)))


def vit_forward_static(handle, d_images, batch, d_tokens, d_taps=None, stream=None):
    return _check("vit_forward_static", lib().vit_forward_static(handle, _ptr(d_images), batch, _ptr(d_tokens),
                                                                 _ptr(d_taps), _stream(stream)))


def vit_descriptor(handle, d_tokens, batch, d_desc, stream=None):
    return _check("vit_descriptor", lib().vit_descriptor(handle, _ptr(d_tokens), batch, _ptr(d_desc),
                                                         _stream(stream)))


def vit_patch_scores(handle, d_image, d_class_emb, classes, mode, d_labels, d_cos=None, d_dense=None, stream=None):
    return _check("vit_patch_scores", lib().vit_patch_scores(
        handle, _ptr(d_image), _ptr(d_class_emb), classes, mode, _ptr(d_labels), _ptr(d_cos), _ptr(d_dense),
        _stream(stream)))


def vit_destroy(handle):
    return _check("vit_destroy", lib().vit_destroy(handle))


def vit_op_linear_residual_ln(a, w, bias, ls, M, N, K, x, g, b, eps, h, stream=None):
    return _check("vit_op_linear_residual_ln",
                  lib().vit_op_linear_residual_ln(_ptr(a), _ptr(w), _ptr(bias), _ptr(ls), M, N, K, _ptr(x), _ptr(g),
                                                  _ptr(b), eps, _ptr(h), _stream(stream)))


def vit_op_preprocess(frames, batch, src_h, src_w, bgr, images, dst_h, dst_w, stream=None):
    return _check("vit_op_preprocess", lib().vit_op_preprocess(_ptr(frames), batch, src_h, src_w, int(bgr),
                                                               _ptr(images), dst_h, dst_w, _stream(stream)))


def vit_op_layernorm(x, rows, dim, g, b, eps, y, out_fp32, stream=None):
    return _check("vit_op_layernorm", lib().vit_op_layernorm(_ptr(x), rows, dim, _ptr(g), _ptr(b), eps, _ptr(y),
                                                             int(out_fp32), _stream(stream)))


def vit_op_linear(a, w, bias, M, N, K, epilogue, ls, c, stream=None):
    return _check("vit_op_linear", lib().vit_op_linear(_ptr(a), _ptr(w), _ptr(bias), M, N, K, epilogue, _ptr(ls),
                                                       _ptr(c), _stream(stream)))


def vit_op_qkv(h, wqkv, bqkv, batch, tokens, heads, q, k, vt, stream=None):
    return _check("vit_op_qkv", lib().vit_op_qkv(_ptr(h), _ptr(wqkv), _ptr(bqkv), batch, tokens, heads, _ptr(q),
                                                 _ptr(k), _ptr(vt), _stream(stream)))


def vit_op_attention(q, k, vt, batch, tokens, heads, o, stream=None):
    return _check("vit_op_attention", lib().vit_op_attention(_ptr(q), _ptr(k), _ptr(vt), batch, tokens, heads,
                                                             _ptr(o), _stream(stream)))


# ------------------------------------------------------------------ marshalling helpers

def config_from_dict(cfg: dict, max_batch: int | None = None) -> VitConfig:
    """A VitConfig from a workload dictionary (keys as in the seeded-input presets)."""
    gh, gw = cfg.get("pos_grid") or (cfg["img_h"] // cfg["patch"], cfg["img_w"] // cfg["patch"])
    mask = 0
    for t in cfg.get("taps", ()):
        mask |= 1 << (t - 1)
    mb = max_batch if max_batch is not None else max(cfg.get("batches", (1,)))
    return VitConfig(cfg["img_h"], cfg["img_w"], cfg["patch"], cfg["dim"], cfg["depth"], cfg.get("extra_blocks", 0),
                     cfg["heads"], cfg["mlp_hidden"], cfg["registers"], mb, cfg["ln_eps"], mask, gh, gw,
                     cfg.get("window", 0), cfg.get("window_stride", 0), cfg.get("classes", 0))


_BLOCK_ORDER = ("ln1_g", "ln1_b", "wq", "bq", "wk", "bk", "wv", "bv", "wo", "bo", "ls1", "ln2_g", "ln2_b",
                "w1", "b1", "w2", "b2", "ls2")


def pack_params(P: dict) -> np.ndarray:
    """Concatenate a parameter dictionary into the fp32 blob order of vit_create."""
    parts = [P["patch_w"], P["patch_b"], P["cls"], P["reg"], P["pos"]]
    for b in P["blocks"]:
        parts.extend(b[k] for k in _BLOCK_ORDER)
    parts.extend([P["norm_g"], P["norm_b"]])
    return np.concatenate([np.ascontiguousarray(a, dtype=np.float32).ravel() for a in parts])


class Encoder:
    """A created model with torch-owned weight and workspace buffers on one device."""

    def __init__(self, cfg: dict | VitConfig, params: dict | np.ndarray, max_batch: int | None = None,
                 device: str = "cuda", stream=None, workspace: bool = True):
        """workspace=False binds no workspace: only forward_static can run."""
        import torch
        self.cfg = cfg if isinstance(cfg, VitConfig) else config_from_dict(cfg, max_batch)
        self.sizes = vit_plan(self.cfg)
        blob = params if isinstance(params, np.ndarray) else pack_params(params)
        self.device = torch.device(device)
        self.weights = torch.empty(self.sizes.weight_bytes, dtype=torch.uint8, device=self.device)
        self.workspace = (torch.empty(self.sizes.workspace_bytes, dtype=torch.uint8, device=self.device)
                          if workspace else None)
        self.handle = vit_create(self.cfg, blob, self.weights, self.workspace, stream)

    @property
    def tokens(self) -> int:
        return self.sizes.tokens

    def forward(self, images, with_taps: bool = False, tokens_out=None, taps_out=None, stream=None):
        import torch
        B = images.shape[0]
        c = self.cfg
        if tokens_out is None:
            tokens_out = torch.empty((B, self.sizes.tokens, c.dim), dtype=torch.float32, device=self.device)
        if with_taps and taps_out is None:
            taps_out = torch.empty((B, self.sizes.taps, c.dim, c.img_h // c.patch, c.img_w // c.patch),
                                   dtype=torch.float32, device=self.device)
        vit_forward(self.handle, images, B, tokens_out, taps_out if with_taps else None, stream)
        return (tokens_out, taps_out) if with_taps else tokens_out

    def forward_static(self, images, with_taps: bool = False, tokens_out=None, taps_out=None, stream=None):
        """forward() with the activations in the library's static device array
        (vit_forward_static): the library allocates nothing; the outputs are
        torch buffers made here unless given."""
        import torch
        B = images.shape[0]
        c = self.cfg
        if tokens_out is None:
            tokens_out = torch.empty((B, self.sizes.tokens, c.dim), dtype=torch.float32, device=self.device)
        if with_taps and taps_out is None:
            taps_out = torch.empty((B, self.sizes.taps, c.dim, c.img_h // c.patch, c.img_w // c.patch),
                                   dtype=torch.float32, device=self.device)
        vit_forward_static(self.handle, images, B, tokens_out, taps_out if with_taps else None, stream)
        return (tokens_out, taps_out) if with_taps else tokens_out

    def descriptor(self, tokens, desc_out=None, stream=None):
        import torch
        B = tokens.shape[0]
        if desc_out is None:
            desc_out = torch.empty((B, self.cfg.dim), dtype=torch.float32, device=self.device)
        vit_descriptor(self.handle, tokens, B, desc_out, stream)
        return desc_out

    def patch_scores(self, image, class_emb, mode: int, want_cos: bool = False, want_dense: bool = False,
                     stream=None):
        import torch
        c = self.cfg
        C = class_emb.shape[0]
        labels = torch.empty((c.img_h, c.img_w), dtype=torch.int32, device=self.device)
        cos = dense = None
        p = c.patch
        if want_cos:
            if mode == 0:
                cos = torch.empty((C, c.img_h // p, c.img_w // p), dtype=torch.float32, device=self.device)
            else:
                g = c.window // p
                cos = torch.empty((self.sizes.windows, C, g, g), dtype=torch.float32, device=self.device)
        if want_dense:
            dense = torch.empty((C, c.img_h, c.img_w), dtype=torch.float32, device=self.device)
        vit_patch_scores(self.handle, image, class_emb, C, mode, labels, cos, dense, stream)
        return labels, cos, dense

    def close(self):
        if getattr(self, "handle", None) is not None:
            vit_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class EncoderGraph:
    """One ``Encoder.forward`` (and optionally ``descriptor``) over fixed device
    buffers, recorded once as a HIP graph; ``replay()`` enqueues the whole
    forward as a single graph launch on the current stream.  New inputs are
    written into ``images`` in place between replays.  The forward enqueues
    kernels only (no allocation, copy, memset or host synchronisation), which
    is what makes it capturable."""

    def __init__(self, enc: Encoder, images, tokens_out, desc_out=None, taps_out=None):
        import torch
        self.enc, self.images, self.tokens, self.desc, self.taps = enc, images, tokens_out, desc_out, taps_out
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # one eager run before capture
            self._record()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._record()

    def _record(self):
        self.enc.forward(self.images, with_taps=self.taps is not None, tokens_out=self.tokens, taps_out=self.taps)
        if self.desc is not None:
            self.enc.descriptor(self.tokens, desc_out=self.desc)

    def replay(self):
        self.graph.replay()



# ---------------------------------------------------------------------------- semantic head

class HeadConfig(ctypes.Structure):
    """Mirror of vit_head_config (include/vit_head.h)."""
    _fields_ = [("grid_h", _I), ("grid_w", _I), ("dim", _I), ("taps", _I), ("width", _I), ("groups", _I),
                ("classes", _I), ("out_h", _I), ("out_w", _I), ("max_batch", _I), ("ln_eps", ctypes.c_float),
                ("gn_eps", ctypes.c_float)]


class HeadSizes(ctypes.Structure):
    """Mirror of vit_head_sizes."""
    _fields_ = [("weight_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t),
                ("host_floats", ctypes.c_size_t)]


def head_config_preset() -> HeadConfig:
    c = HeadConfig()
    _check("vit_head_config_preset", lib().vit_head_config_preset(ctypes.byref(c)))
    return c


def head_config(grid_h: int, grid_w: int, out_h: int, out_w: int, max_batch: int, dim: int = 384, taps: int = 4,
                width: int = 256, classes: int = 19) -> HeadConfig:
    """A HeadConfig for the given geometry (the diagram's widths and epsilons otherwise)."""
    return HeadConfig(grid_h, grid_w, dim, taps, width, width // 8, classes, out_h, out_w, max_batch, 1e-6, 1e-5)


def head_plan(cfg: HeadConfig) -> HeadSizes:
    s = HeadSizes()
    _check("vit_head_plan", lib().vit_head_plan(ctypes.byref(cfg), ctypes.byref(s)))
    return s


_HEAD_ORDER = (["proj_w", "proj_ln_g", "proj_ln_b"]
               + [f"bn{i}_{k}" for i in (1, 2, 3) for k in ("w1", "ln1_g", "ln1_b", "w2", "ln2_g", "ln2_b")]
               + ["out_w", "out_ln_g", "out_ln_b", "final_ln_g", "final_ln_b", "lat_w", "lat_b", "smooth_w",
                  "smooth_b", "gn_g", "gn_b", "pred_w", "pred_b"])


def pack_head_params(P: dict) -> np.ndarray:
    """Concatenate a head parameter dictionary into the fp32 blob order of vit_head_create."""
    return np.concatenate([np.ascontiguousarray(P[k], dtype=np.float32).ravel() for k in _HEAD_ORDER])


def vit_op_conv3x3(x, ld_in, c0, cin, batch, gh, gw, w, bias, n_out, out, stream=None):
    return _check("vit_op_conv3x3", lib().vit_op_conv3x3(_ptr(x), ld_in, c0, cin, batch, gh, gw, _ptr(w), _ptr(bias),
                                                         n_out, _ptr(out), _stream(stream)))


def vit_op_convx(x, ld_in, c0, cin, batch, gh, gw, ksize, w, n_out, g, b, g2, b2, eps, out, ld_out, c0_out,
                 stream=None):
    return _check("vit_op_convx", lib().vit_op_convx(_ptr(x), ld_in, c0, cin, batch, gh, gw, ksize, _ptr(w), n_out,
                                                     _ptr(g), _ptr(b), _ptr(g2), _ptr(b2), eps, _ptr(out), ld_out,
                                                     c0_out, _stream(stream)))


def vit_op_absmax(x, n, amax, stream=None):
    import torch
    return _check("vit_op_absmax", lib().vit_op_absmax(_ptr(x), int(x.dtype == torch.bfloat16), n, _ptr(amax),
                                                       _stream(stream)))


def vit_op_quantize_fp8(x, n, s_inv, out, stream=None):
    import torch
    return _check("vit_op_quantize_fp8", lib().vit_op_quantize_fp8(_ptr(x), int(x.dtype == torch.bfloat16), n, s_inv,
                                                                   _ptr(out), _stream(stream)))


def vit_op_linear_fp8(a, w, M, N, K, scale, bias, out, stream=None):
    import torch
    return _check("vit_op_linear_fp8", lib().vit_op_linear_fp8(_ptr(a), _ptr(w), M, N, K, scale, _ptr(bias), _ptr(out),
                                                               int(out.dtype == torch.float32), _stream(stream)))


def vit_op_quantize_int8(x, n, s_inv, out, stream=None):
    import torch
    return _check("vit_op_quantize_int8", lib().vit_op_quantize_int8(_ptr(x), int(x.dtype == torch.bfloat16), n, s_inv,
                                                                     _ptr(out), _stream(stream)))


def vit_op_linear_int8(a, w, M, N, K, scale, bias, out, stream=None):
    import torch
    return _check("vit_op_linear_int8", lib().vit_op_linear_int8(_ptr(a), _ptr(w), M, N, K, scale, _ptr(bias),
                                                                 _ptr(out), int(out.dtype == torch.float32),
                                                                 _stream(stream)))


class SemanticHead:
    """A created semantic head with torch-owned weight and workspace buffers."""

    def __init__(self, cfg: HeadConfig, params: dict | np.ndarray, device: str = "cuda", stream=None):
        import torch
        self.cfg = cfg
        self.sizes = head_plan(cfg)
        blob = params if isinstance(params, np.ndarray) else pack_head_params(params)
        self.device = torch.device(device)
        self.weights = torch.empty(self.sizes.weight_bytes, dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(self.sizes.workspace_bytes, dtype=torch.uint8, device=self.device)
        blob = np.ascontiguousarray(blob, dtype=np.float32)
        h = _P()
        _check("vit_head_create", lib().vit_head_create(ctypes.byref(cfg), blob.ctypes.data, blob.size,
                                                        _ptr(self.weights), self.sizes.weight_bytes,
                                                        _ptr(self.workspace), self.sizes.workspace_bytes,
                                                        _stream(stream), ctypes.byref(h)))
        self.handle = h

    def forward(self, taps, logits_out=None, want_grid: bool = False, stream=None):
        import torch
        c = self.cfg
        B = taps.shape[0]
        if logits_out is None:
            logits_out = torch.empty((B, c.classes, c.out_h, c.out_w), dtype=torch.float32, device=self.device)
        grid = None
        if want_grid:
            grid = torch.empty((B, c.classes, c.grid_h, c.grid_w), dtype=torch.float32, device=self.device)
        _check("vit_head_forward", lib().vit_head_forward(self.handle, _ptr(taps), B, _ptr(logits_out), _ptr(grid),
                                                          _stream(stream)))
        return (logits_out, grid) if want_grid else logits_out

    def close(self):
        if getattr(self, "handle", None) is not None:
            lib().vit_head_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
