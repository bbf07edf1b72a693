"""wav2vec2-CTC encoder inference on AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libw2v2.so`` (include/w2v2.h).  It
only marshals arguments: device buffers are torch tensors (their
``data_ptr()``), the stream is torch's current HIP stream, and every step of
the network runs in the library's HIP kernels.  There is no fallback: if the
library is missing or the device is not a gfx950, calls raise.

    model = Model(cfg, weights)             # cfg: object or dict with the config fields
    logits, vframes = model.forward(pcm, valid)   # cuda fp32 [B, W], cuda int32 [B]
    ids, lens = ctc_greedy(logits, vframes, blank_id=cfg.blank_id)
"""
from __future__ import annotations

import ctypes
from typing import Any, Mapping

import numpy as np
import torch

from . import _lib
from ._lib import W2V2Error, LibraryMissing  # noqa: F401

__all__ = ["Model", "ctc_greedy", "W2V2Error", "LibraryMissing", "make_config", "amax_table", "FP8_INPUTS"]

# inputs of the fp8 mode's projections, in the order of w2v2_calibrate's slots
FP8_INPUTS = ("attn.qkv", "attn.out", "ffn.fc1", "ffn.fc2")


def amax_table(amax) -> dict:
    """Weight-table entries {layer{l}.<input>.input_amax: fp32 [1]} of an fp8
    model from a calibration result [layers, 4] (tensor or array)."""
    a = np.asarray(amax.cpu() if isinstance(amax, torch.Tensor) else amax, dtype=np.float32)
    return {f"layer{l}.{w}.input_amax": np.array([a[l, k]], np.float32)
            for l in range(a.shape[0]) for k, w in enumerate(FP8_INPUTS)}


def _get(cfg: Any, name: str, default=None):
    if isinstance(cfg, Mapping):
        return cfg.get(name, default)
    return getattr(cfg, name, default)


def make_config(cfg: Any, max_batch: int | None = None, precision: str | None = None) -> _lib.Config:
    """C config struct from an object or mapping with the fields of
    ``w2v2_config`` (conv_dim, conv_kernel, conv_stride, conv_bias,
    feat_norm "group"/"layer", hidden, heads, ffn, layers, pos_kernel,
    pos_groups, stable_layer_norm, vocab, blank_id, eps, precision
    "fp32"/"fp16", window, batch, gelu "erf"/"tanh")."""
    c = _lib.Config()
    c.abi_version = _lib.ABI_VERSION
    c.sample_rate = int(_get(cfg, "sample_rate", 16000))
    dims, ks, ss = list(_get(cfg, "conv_dim")), list(_get(cfg, "conv_kernel")), list(_get(cfg, "conv_stride"))
    if not (len(dims) == len(ks) == len(ss)) or len(dims) > _lib.MAX_CONV:
        raise ValueError("conv_dim, conv_kernel and conv_stride must have the same length <= 8")
    c.n_conv = len(dims)
    for i in range(len(dims)):
        c.conv_dim[i], c.conv_kernel[i], c.conv_stride[i] = int(dims[i]), int(ks[i]), int(ss[i])
    c.conv_bias = int(bool(_get(cfg, "conv_bias", False)))
    fn = _get(cfg, "feat_norm", "group")
    c.feat_norm = {"group": 0, "layer": 1}[fn] if isinstance(fn, str) else int(fn)
    for f in ("hidden", "heads", "ffn", "layers", "pos_kernel", "pos_groups", "vocab"):
        setattr(c, f, int(_get(cfg, f)))
    c.blank_id = int(_get(cfg, "blank_id", 0))
    c.stable_layer_norm = int(bool(_get(cfg, "stable_layer_norm", False)))
    c.eps = float(_get(cfg, "eps", 1e-5))
    prec = precision if precision is not None else _get(cfg, "precision", "fp16")
    c.precision = ({"fp32": 0, "fp16": 1, "fp8": 2, "fp8_on_fp32": 3}[prec] if isinstance(prec, str)
                   else int(prec))
    c.max_batch = int(max_batch if max_batch is not None else _get(cfg, "batch", 1))
    c.window = int(_get(cfg, "window"))
    g = _get(cfg, "gelu", "erf")
    c.gelu_kind = {"erf": 0, "tanh": 1}[g] if isinstance(g, str) else int(g)
    return c


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, dtype: torch.dtype, shape: tuple, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


class Model:
    """One network on one GPU (``w2v2_create`` / ``w2v2_destroy``)."""

    def __init__(self, cfg: Any, weights: Mapping[str, np.ndarray], device: int = 0,
                 max_batch: int | None = None, precision: str | None = None):
        L = _lib.lib()
        self._cfg = make_config(cfg, max_batch=max_batch, precision=precision)
        arrays = {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in weights.items()}
        names = [k.encode() for k in arrays]
        tab = (_lib.Tensor * max(1, len(arrays)))()
        for i, (k, a) in enumerate(arrays.items()):
            tab[i].name = names[i]
            tab[i].data = a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
            tab[i].ndim = a.ndim
            for j, s in enumerate(a.shape[:4]):
                tab[i].shape[j] = s
        h = ctypes.c_void_p()
        self._h = None
        _lib.check(L.w2v2_create(ctypes.byref(self._cfg), tab, len(arrays), int(device), ctypes.byref(h)),
                   "w2v2_create")
        self._h = h
        self.device = torch.device("cuda", int(device))
        t, v, ws = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
        _lib.check(L.w2v2_model_info(h, ctypes.byref(t), ctypes.byref(v), ctypes.byref(ws)), "w2v2_model_info")
        self.frames_per_window, self.vocab, self.workspace_bytes = t.value, v.value, ws.value
        self.max_batch = self._cfg.max_batch
        self.window = self._cfg.window
        self.conv_dim_last = self._cfg.conv_dim[self._cfg.n_conv - 1]
        self.blank_id = self._cfg.blank_id

    # -- lifetime --------------------------------------------------------
    def close(self) -> None:
        if self._h is not None:
            torch.cuda.synchronize(self.device)
            _lib.lib().w2v2_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            if self._h is not None:
                _lib.lib().w2v2_destroy(self._h)
                self._h = None
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- host helpers ----------------------------------------------------
    def num_frames(self, samples: int) -> int:
        out = ctypes.c_int32()
        _lib.check(_lib.lib().w2v2_num_frames(self._h, int(samples), ctypes.byref(out)), "w2v2_num_frames")
        return out.value

    # -- device calls ----------------------------------------------------
    def forward(self, pcm: torch.Tensor, valid: torch.Tensor, logits: torch.Tensor | None = None,
                vframes: torch.Tensor | None = None, stream=None):
        B = pcm.shape[0]
        _need(pcm, torch.float32, (B, self.window), "pcm")
        _need(valid, torch.int32, (B,), "valid")
        if logits is None:
            logits = torch.empty(B, self.frames_per_window, self.vocab, dtype=torch.float32, device=pcm.device)
        if vframes is None:
            vframes = torch.empty(B, dtype=torch.int32, device=pcm.device)
        _need(logits, torch.float32, (B, self.frames_per_window, self.vocab), "logits")
        _need(vframes, torch.int32, (B,), "vframes")
        _lib.check(_lib.lib().w2v2_forward(self._h, _ptr(pcm), _ptr(valid), B, _ptr(logits), _ptr(vframes),
                                           _stream(stream)), "w2v2_forward")
        return logits, vframes

    def forward_greedy(self, pcm: torch.Tensor, valid: torch.Tensor, logits: torch.Tensor | None = None,
                       vframes: torch.Tensor | None = None, ids: torch.Tensor | None = None,
                       lens: torch.Tensor | None = None, stream=None):
        """Forward plus greedy CTC decoding in one call (``w2v2_forward_greedy``):
        the CTC head's epilogue takes each frame's argmax, so the logits are not
        read again.  Returns (logits, vframes, ids, lens)."""
        B = pcm.shape[0]
        _need(pcm, torch.float32, (B, self.window), "pcm")
        _need(valid, torch.int32, (B,), "valid")
        T = self.frames_per_window
        dev = pcm.device
        logits = torch.empty(B, T, self.vocab, dtype=torch.float32, device=dev) if logits is None else logits
        vframes = torch.empty(B, dtype=torch.int32, device=dev) if vframes is None else vframes
        ids = torch.empty(B, T, dtype=torch.int32, device=dev) if ids is None else ids
        lens = torch.empty(B, dtype=torch.int32, device=dev) if lens is None else lens
        _need(logits, torch.float32, (B, T, self.vocab), "logits")
        _need(vframes, torch.int32, (B,), "vframes")
        _need(ids, torch.int32, (B, T), "ids")
        _need(lens, torch.int32, (B,), "lens")
        _lib.check(_lib.lib().w2v2_forward_greedy(self._h, _ptr(pcm), _ptr(valid), B, _ptr(logits), _ptr(vframes),
                                                  _ptr(ids), _ptr(lens), _stream(stream)), "w2v2_forward_greedy")
        return logits, vframes, ids, lens

    def forward_greedy_noalloc(self, pcm: torch.Tensor, valid: torch.Tensor, logits: torch.Tensor,
                               vframes: torch.Tensor, ids: torch.Tensor, lens: torch.Tensor, stream=None):
        """forward_greedy with every intermediate in the library's static
        device scratch (``w2v2_forward_greedy_noalloc``): the caller passes
        all outputs, nothing is allocated."""
        B = pcm.shape[0]
        T = self.frames_per_window
        _need(pcm, torch.float32, (B, self.window), "pcm")
        _need(valid, torch.int32, (B,), "valid")
        _need(logits, torch.float32, (B, T, self.vocab), "logits")
        _need(vframes, torch.int32, (B,), "vframes")
        _need(ids, torch.int32, (B, T), "ids")
        _need(lens, torch.int32, (B,), "lens")
        _lib.check(_lib.lib().w2v2_forward_greedy_noalloc(self._h, _ptr(pcm), _ptr(valid), B, _ptr(logits),
                                                          _ptr(vframes), _ptr(ids), _ptr(lens), _stream(stream)),
                   "w2v2_forward_greedy_noalloc")
        return logits, vframes, ids, lens

    def forward_true_length(self, pcm: torch.Tensor, valid, logits: torch.Tensor | None = None,
                            vframes: torch.Tensor | None = None, stream=None):
        """Every row as its own true-length clip of valid[b] samples.

        ``valid`` is a host array (numpy or CPU tensor) of int32 sample counts;
        the library reads it during the call.  Frames past a row's own frame
        count come back as 0."""
        B = pcm.shape[0]
        _need(pcm, torch.float32, (B, self.window), "pcm")
        vh = np.ascontiguousarray(np.asarray(valid.cpu() if isinstance(valid, torch.Tensor) else valid,
                                             dtype=np.int32))
        if vh.shape != (B,):
            raise ValueError(f"valid: expected host int32 [{B}], got shape {vh.shape}")
        if logits is None:
            logits = torch.empty(B, self.frames_per_window, self.vocab, dtype=torch.float32, device=pcm.device)
        if vframes is None:
            vframes = torch.empty(B, dtype=torch.int32, device=pcm.device)
        _need(logits, torch.float32, (B, self.frames_per_window, self.vocab), "logits")
        _need(vframes, torch.int32, (B,), "vframes")
        _lib.check(_lib.lib().w2v2_forward_true_length(self._h, _ptr(pcm), vh.ctypes.data, B, _ptr(logits),
                                                       _ptr(vframes), _stream(stream)), "w2v2_forward_true_length")
        return logits, vframes

    def forward_frontend(self, pcm: torch.Tensor, valid: torch.Tensor, features: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
        B = pcm.shape[0]
        _need(pcm, torch.float32, (B, self.window), "pcm")
        _need(valid, torch.int32, (B,), "valid")
        shape = (B, self.frames_per_window, self.conv_dim_last)
        if features is None:
            features = torch.empty(shape, dtype=torch.float32, device=pcm.device)
        _need(features, torch.float32, shape, "features")
        _lib.check(_lib.lib().w2v2_forward_frontend(self._h, _ptr(pcm), _ptr(valid), B, _ptr(features),
                                                    _stream(stream)), "w2v2_forward_frontend")
        return features

    def forward_encoder(self, features: torch.Tensor, logits: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
        B = features.shape[0]
        _need(features, torch.float32, (B, self.frames_per_window, self.conv_dim_last), "features")
        if logits is None:
            logits = torch.empty(B, self.frames_per_window, self.vocab, dtype=torch.float32,
                                 device=features.device)
        _need(logits, torch.float32, (B, self.frames_per_window, self.vocab), "logits")
        _lib.check(_lib.lib().w2v2_forward_encoder(self._h, _ptr(features), B, _ptr(logits), _stream(stream)),
                   "w2v2_forward_encoder")
        return logits

    def calibrate(self, pcm: torch.Tensor, valid: torch.Tensor, amax: torch.Tensor | None = None,
                  logits: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """Raise amax (cuda fp32 [layers, 4], zero-filled here if not given) to
        the max |x| at the inputs of every block's q/k/v, out, fc1 and fc2
        projections over this batch (``w2v2_calibrate``)."""
        B = pcm.shape[0]
        _need(pcm, torch.float32, (B, self.window), "pcm")
        _need(valid, torch.int32, (B,), "valid")
        if amax is None:
            amax = torch.zeros(self._cfg.layers, 4, dtype=torch.float32, device=pcm.device)
        _need(amax, torch.float32, (self._cfg.layers, 4), "amax")
        if logits is None:
            logits = torch.empty(B, self.frames_per_window, self.vocab, dtype=torch.float32, device=pcm.device)
        _lib.check(_lib.lib().w2v2_calibrate(self._h, _ptr(pcm), _ptr(valid), B, _ptr(logits), _ptr(amax),
                                             _stream(stream)), "w2v2_calibrate")
        return amax

    # -- kernel timing ---------------------------------------------------
    def profile_enable(self, on: bool = True, only: str | None = None) -> None:
        """Time every kernel launch (or only launches of kernel ``only``) with HIP events."""
        _lib.check(_lib.lib().w2v2_profile_enable(self._h, int(bool(on)), None if only is None else only.encode()),
                   "w2v2_profile_enable")

    def profile_read(self) -> dict[str, tuple[float, int]]:
        """{kernel name: (total ms, launches)} since the previous read."""
        cap = 64
        names = (ctypes.c_char_p * cap)()
        ms = (ctypes.c_double * cap)()
        cnt = (ctypes.c_int64 * cap)()
        n = ctypes.c_int32()
        _lib.check(_lib.lib().w2v2_profile_read(self._h, cap, names, ms, cnt, ctypes.byref(n)), "w2v2_profile_read")
        return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n.value, cap))}


def ctc_greedy(logits: torch.Tensor, vframes: torch.Tensor, blank_id: int = 0, ids: torch.Tensor | None = None,
               lens: torch.Tensor | None = None, stream=None):
    """Greedy CTC decoding on the device (``w2v2_ctc_greedy``).

    Returns (ids int32 [B, T] with -1 after each row's tokens, lens int32 [B])."""
    B, T, V = logits.shape
    _need(logits, torch.float32, (B, T, V), "logits")
    _need(vframes, torch.int32, (B,), "vframes")
    if ids is None:
        ids = torch.empty(B, T, dtype=torch.int32, device=logits.device)
    if lens is None:
        lens = torch.empty(B, dtype=torch.int32, device=logits.device)
    _need(ids, torch.int32, (B, T), "ids")
    _need(lens, torch.int32, (B,), "lens")
    _lib.check(_lib.lib().w2v2_ctc_greedy(_ptr(logits), _ptr(vframes), B, T, V, int(blank_id), _ptr(ids),
                                          _ptr(lens), _stream(stream)), "w2v2_ctc_greedy")
    return ids, lens
