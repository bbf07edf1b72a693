"""Seeded synthetic inputs for wav2vec2-CTC encoder inference.

This module is shared by the CPU oracle (``oracle/``), the HIP library's
Python binding, the tests and the benchmark.  It holds *only* input
descriptions: the five workload presets (shapes and sizes), the parameter
inventory with its seeded initial values, and seeded 16 kHz PCM with valid
lengths.  It contains none of the network's arithmetic; both the oracle and
the GPU path receive exactly the arrays produced here.

Value recipes (all draws from ``numpy.random.default_rng(seed)``):

* weights: every weight matrix and conv kernel ~ N(0, 0.02); biases 0; norm
  gains 1 and shifts 0; weight-norm gains g = 1.  With ``rand_affine=True``
  (the tiny preset, and the parity tests that exercise every affine path)
  biases ~ N(0, 0.02), norm gains ~ 1 + N(0, 0.1), shifts ~ N(0, 0.05) and
  weight-norm gains ~ U[0.5, 1.5].
* PCM "sines": three sines with f ~ U[100, 3000] Hz, random phase, amplitude
  0.3 each, plus N(0, 0.05) noise.
* PCM "speech": consecutive 150-300 ms segments, 15% silent, the rest a
  harmonic stack (f0 ~ U[90, 250] Hz, harmonics k*f0 <= 4 kHz with amplitude
  1/k, random phases) under a sin^2 envelope; scaled to peak 0.3, plus
  N(0, 0.05) noise.  Samples at or beyond a row's valid length are 0 (the
  window is zero-padded) unless ``pad_garbage`` asks for noise there.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

SAMPLE_RATE = 16000


@dataclass(frozen=True)
class W2V2Config:
    """Shape description of one wav2vec2-CTC network plus its workload."""

    name: str = "custom"
    conv_dim: tuple = (512,) * 7
    conv_kernel: tuple = (10, 3, 3, 3, 3, 2, 2)
    conv_stride: tuple = (5, 2, 2, 2, 2, 2, 2)
    conv_bias: bool = False
    feat_norm: str = "group"          # "group" (layer 0 only) | "layer" (every conv)
    hidden: int = 768
    heads: int = 12
    ffn: int = 3072
    layers: int = 12
    pos_kernel: int = 128
    pos_groups: int = 16
    stable_layer_norm: bool = False   # False: post-norm blocks; True: pre-norm + final LN
    vocab: int = 32
    blank_id: int = 0
    eps: float = 1e-5
    gelu: str = "erf"                 # "erf" (exact) | "tanh" (tanh approximation)
    precision: str = "fp16"           # "fp32" | "fp16" (fp16 operands, fp32 accumulate/normalise)
    window: int = 256000              # samples per window
    batch: int = 8
    valid_range: tuple | None = None  # (lo, hi) samples, inclusive; None = full window
    pcm_kind: str = "speech"          # "speech" | "sines"
    weight_seed: int = 1234
    pcm_seed: int = 100
    rand_affine: bool = False

    def replace(self, **kw) -> "W2V2Config":
        return dataclasses.replace(self, **kw)


# The five workloads.  Names state what they are.
TINY_1S_B1 = W2V2Config(
    name="tiny_1s_b1", conv_dim=(32,) * 7, hidden=64, heads=4, ffn=256, layers=2,
    pos_kernel=16, pos_groups=4, vocab=32, precision="fp32", window=16000, batch=1,
    pcm_kind="sines", weight_seed=1235, pcm_seed=101, rand_affine=True)
BASE_10S_B1 = W2V2Config(
    name="base_10s_b1", window=160000, batch=1, weight_seed=1236, pcm_seed=201)
BASE_16S_B8 = W2V2Config(
    name="base_16s_b8", window=256000, batch=8, valid_range=(32000, 256000),
    weight_seed=1237, pcm_seed=301)
LARGE_16S_B4 = W2V2Config(
    name="large_16s_b4", conv_bias=True, feat_norm="layer", hidden=1024, heads=16,
    ffn=4096, layers=24, stable_layer_norm=True, vocab=2341, window=256000, batch=4,
    weight_seed=1238, pcm_seed=401)
BASE_16S_B32 = W2V2Config(
    name="base_16s_b32", window=256000, batch=32, valid_range=(16000, 256000),
    weight_seed=1239, pcm_seed=501)

PRESETS = {c.name: c for c in (TINY_1S_B1, BASE_10S_B1, BASE_16S_B8, LARGE_16S_B4, BASE_16S_B32)}


# ----------------------------------------------------------------------------
# parameter inventory
# ----------------------------------------------------------------------------
def weight_shapes(cfg: W2V2Config) -> list[tuple[str, tuple, str]]:
    """Ordered (name, shape, kind) for every parameter of ``cfg``.

    kind is one of "w" (matrix / kernel), "b" (bias), "gamma", "beta",
    "wn_v" and "wn_g" (weight-norm direction and per-tap gain).
    Shapes follow the usual PyTorch conventions: conv kernels are
    [C_out, C_in / groups, K], linear weights are [out, in].
    """
    out: list[tuple[str, tuple, str]] = []
    c_in = 1
    for i, (c, k) in enumerate(zip(cfg.conv_dim, cfg.conv_kernel)):
        out.append((f"fe.conv{i}.weight", (c, c_in, k), "w"))
        if cfg.conv_bias:
            out.append((f"fe.conv{i}.bias", (c,), "b"))
        if cfg.feat_norm == "layer" or i == 0:
            out.append((f"fe.norm{i}.weight", (c,), "gamma"))
            out.append((f"fe.norm{i}.bias", (c,), "beta"))
        c_in = c
    d, c_last = cfg.hidden, cfg.conv_dim[-1]
    out += [("fp.norm.weight", (c_last,), "gamma"), ("fp.norm.bias", (c_last,), "beta"),
            ("fp.proj.weight", (d, c_last), "w"), ("fp.proj.bias", (d,), "b"),
            ("pos.weight_v", (d, d // cfg.pos_groups, cfg.pos_kernel), "wn_v"),
            ("pos.weight_g", (cfg.pos_kernel,), "wn_g"),
            ("pos.bias", (d,), "b"),
            ("enc.norm.weight", (d,), "gamma"), ("enc.norm.bias", (d,), "beta")]
    for l in range(cfg.layers):
        p = f"layer{l}."
        for proj in ("q", "k", "v", "out"):
            out += [(p + f"attn.{proj}.weight", (d, d), "w"), (p + f"attn.{proj}.bias", (d,), "b")]
        out += [(p + "attn_norm.weight", (d,), "gamma"), (p + "attn_norm.bias", (d,), "beta"),
                (p + "ffn.fc1.weight", (cfg.ffn, d), "w"), (p + "ffn.fc1.bias", (cfg.ffn,), "b"),
                (p + "ffn.fc2.weight", (d, cfg.ffn), "w"), (p + "ffn.fc2.bias", (d,), "b"),
                (p + "ffn_norm.weight", (d,), "gamma"), (p + "ffn_norm.bias", (d,), "beta")]
    out += [("head.weight", (cfg.vocab, d), "w"), ("head.bias", (cfg.vocab,), "b")]
    return out


def make_weights(cfg: W2V2Config, seed: int | None = None,
                 rand_affine: bool | None = None) -> dict[str, np.ndarray]:
    """Seeded host fp32 weight table {name: array} (unfolded weight norm)."""
    rng = np.random.default_rng(cfg.weight_seed if seed is None else seed)
    ra = cfg.rand_affine if rand_affine is None else rand_affine
    w: dict[str, np.ndarray] = {}
    for name, shape, kind in weight_shapes(cfg):
        n = int(np.prod(shape))
        if kind in ("w", "wn_v"):
            a = rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
        elif kind == "b":
            a = (rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)
                 if ra else np.zeros(n, np.float32))
        elif kind == "gamma":
            a = (np.float32(1) + rng.standard_normal(n, dtype=np.float32) * np.float32(0.1)
                 if ra else np.ones(n, np.float32))
        elif kind == "beta":
            a = (rng.standard_normal(n, dtype=np.float32) * np.float32(0.05)
                 if ra else np.zeros(n, np.float32))
        elif kind == "wn_g":
            a = (rng.uniform(0.5, 1.5, n).astype(np.float32) if ra else np.ones(n, np.float32))
        else:  # pragma: no cover
            raise ValueError(kind)
        w[name] = np.ascontiguousarray(a.reshape(shape))
    return w


# ----------------------------------------------------------------------------
# PCM
# ----------------------------------------------------------------------------
def _sines(rng: np.random.Generator, n: int) -> np.ndarray:
    t = np.arange(n, dtype=np.float64) / SAMPLE_RATE
    x = np.zeros(n, np.float64)
    for _ in range(3):
        f = rng.uniform(100.0, 3000.0)
        ph = rng.uniform(0.0, 2 * np.pi)
        x += 0.3 * np.sin(2 * np.pi * f * t + ph)
    return x + rng.normal(0.0, 0.05, n)


def _speech_like(rng: np.random.Generator, n: int) -> np.ndarray:
    x = np.zeros(n, np.float64)
    pos = 0
    while pos < n:
        seg = min(int(rng.uniform(0.150, 0.300) * SAMPLE_RATE), n - pos)
        silent = rng.random() < 0.15
        f0 = rng.uniform(90.0, 250.0)
        if not silent and seg > 0:
            t = np.arange(seg, dtype=np.float64) / SAMPLE_RATE
            env = np.sin(np.pi * np.arange(seg, dtype=np.float64) / seg) ** 2
            kmax = int(4000.0 // f0)
            phases = rng.uniform(0.0, 2 * np.pi, kmax)
            s = np.zeros(seg, np.float64)
            for k in range(1, kmax + 1):
                s += np.sin(2 * np.pi * k * f0 * t + phases[k - 1]) / k
            x[pos:pos + seg] = env * s
        pos += seg
    peak = np.abs(x).max()
    if peak > 0:
        x *= 0.3 / peak
    return x + rng.normal(0.0, 0.05, n)


def make_valid(cfg: W2V2Config, seed: int | None = None) -> np.ndarray:
    """Valid lengths (samples) per row, int32 [B]."""
    rng = np.random.default_rng((cfg.pcm_seed if seed is None else seed) + 7919)
    if cfg.valid_range is None:
        return np.full(cfg.batch, cfg.window, np.int32)
    lo, hi = cfg.valid_range
    return rng.integers(lo, hi, size=cfg.batch, endpoint=True).astype(np.int32)


def make_pcm(cfg: W2V2Config, seed: int | None = None, valid: np.ndarray | None = None,
             pad_garbage: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """Seeded PCM window batch: (pcm fp32 [B, window], valid int32 [B])."""
    s = cfg.pcm_seed if seed is None else seed
    if valid is None:
        valid = make_valid(cfg, s)
    valid = np.asarray(valid, np.int32)
    pcm = np.zeros((cfg.batch, cfg.window), np.float32)
    for b in range(cfg.batch):
        rng = np.random.default_rng(s * 1000 + b)
        row = _sines(rng, cfg.window) if cfg.pcm_kind == "sines" else _speech_like(rng, cfg.window)
        row = row.astype(np.float32)
        v = int(valid[b])
        if pad_garbage:
            row[v:] = rng.normal(0.0, 0.5, cfg.window - v).astype(np.float32)
        else:
            row[v:] = 0.0
        pcm[b] = row
    return pcm, valid
