"""Plain CPU oracle of wav2vec2-CTC encoder inference.

TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
definition that the HIP library is checked against.  Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it; the
product path (the C-ABI library and its Python binding) never does, and this
module imports nothing from that path.

It computes the network exactly as defined, in float64 by default (any
numpy float dtype can be passed to bound its own rounding), with the
feature encoder in [B, C, T] layout and every step written as its textbook
definition.  Library primitives used as steps: ``numpy.matmul`` (a matrix
product) and ``scipy.special.erf``.

Sources (cited by page title and section):

* "litert-community/wav2vec2-base-960h-LiteRT - discussion #1" (Hugging Face):
  sections "Recipe", "Rewrites for the GPU", "fp16 / int8".
* "TensorRT-Model-Connect, families/wav2vec2/README.md": intro "Wav2Vec2 CTC
  layouts", "FP8 quantization study", "Recipe that was measured", "Method",
  "Results".

Where the pages leave a step open, the reading taken is stated at the step.

Parity pins: every function here is pinned by a ``-m "not gpu"`` test
against something other than itself (closed forms, brute-force loops,
invariants, an independent library implementation of the same network);
no function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf


# ----------------------------------------------------------------------------
# elementwise pieces
# ----------------------------------------------------------------------------
def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU, x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)).

    The LiteRT discussion ("Rewrites for the GPU") calls its tanh-GELU rewrite
    the only non-exact step of its export, so the model's own GELU is the
    erf form; it is used for the conv feature encoder, the positional conv
    and the feed-forward block alike.
    """
    x = np.asarray(x)
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(x.dtype.type(2.0))))


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """tanh approximation of GELU, x/2 * (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
    (Hendrycks & Gimpel).  The LiteRT discussion ("Rewrites for the GPU")
    exports the model with this form because the mobile GPU rejects erf; it
    is the compatibility option of the network, not its default."""
    x = np.asarray(x)
    c = np.sqrt(x.dtype.type(2.0) / x.dtype.type(np.pi))
    return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x ** 3)))


def activation(cfg):
    """The GELU flavour a config selects (exact erf unless gelu == "tanh")."""
    return gelu_tanh if getattr(cfg, "gelu", "erf") == "tanh" else gelu


E4M3_MAX = 448.0


def quantize_e4m3(x: np.ndarray) -> np.ndarray:
    """Nearest FP8 e4m3 value of x (returned as float64), ties to the even
    mantissa, saturating at +-448.

    e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; the all-ones
    exponent with mantissa 7 is NaN, so there is no infinity) holds +-2^E (1 +
    m/8) for E = -6 .. 8 and the subnormals +-2^-6 m/8: in [2^E, 2^(E+1)) the
    grid spacing is 2^(E-3), below 2^-6 it is 2^-9, and the largest value is
    2^8 * 1.75 = 448.  TensorRT README, "Recipe that was measured": the FP8
    projections quantize with per-tensor scales of amax / 448, so a value at
    the calibrated maximum maps to 448.  Reading (the pages are silent): values
    beyond +-448 clamp to +-448 (saturating quantization) rather than becoming
    NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                        # a = f 2^e, f in [0.5, 1): floor(log2 a) = e - 1
    E = np.clip(e - 1, -6, 8)
    q = np.ldexp(1.0, E - 3)                  # grid spacing at a's binade (2^-9 for subnormals)
    r = np.minimum(np.round(a / q) * q, E4M3_MAX)   # numpy rounds halves to even
    return np.copysign(r, x)


def layer_norm(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float,
               axis: int = -1) -> np.ndarray:
    """LayerNorm over ``axis``: biased variance, eps inside the square root."""
    mu = x.mean(axis=axis, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=axis, keepdims=True)
    shape = [1] * x.ndim
    shape[axis] = -1
    return (x - mu) / np.sqrt(var + eps) * gamma.reshape(shape) + beta.reshape(shape)


def group_norm_over_time(y: np.ndarray, gamma: np.ndarray, beta: np.ndarray,
                         eps: float) -> np.ndarray:
    """GroupNorm with one group per channel on y [B, C, T].

    TensorRT README, "Results": the feature encoder's first normalization is
    "a group norm over every time step of the clip".  Reading: groups = C,
    so the statistics are per (b, c) over all T frames of the padded window.
    """
    mu = y.mean(axis=2, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=2, keepdims=True)
    return (y - mu) / np.sqrt(var + eps) * gamma[None, :, None] + beta[None, :, None]


# ----------------------------------------------------------------------------
# convolutions
# ----------------------------------------------------------------------------
def conv_out_len(length: int, kernel: int, stride: int) -> int:
    """Frames of an unpadded strided conv: floor((L - K) / s) + 1, 0 if L < K."""
    return 0 if length < kernel else (length - kernel) // stride + 1


def conv1d(x: np.ndarray, w: np.ndarray, b: np.ndarray | None, stride: int) -> np.ndarray:
    """Unpadded strided conv1d on x [B, C_in, L], w [C_out, C_in, K].

    y[b, o, t] = bias[o] + sum_k sum_c w[o, c, k] * x[b, c, s*t + k],
    written as one matrix product per tap k.
    """
    bsz, c_in, length = x.shape
    c_out, c_in_w, kernel = w.shape
    assert c_in == c_in_w
    t_out = conv_out_len(length, kernel, stride)
    y = np.zeros((bsz, c_out, t_out), dtype=x.dtype)
    if t_out == 0:
        return y
    for k in range(kernel):
        # contiguous copies only so that numpy's matmul takes its BLAS path
        xs = np.ascontiguousarray(x[:, :, k:k + stride * (t_out - 1) + 1:stride])   # [B, C_in, T]
        y += np.matmul(np.ascontiguousarray(w[:, :, k]), xs)                          # [C_out, C_in] @ [B, C_in, T]
    if b is not None:
        y += b[None, :, None]
    return y


def fold_weight_norm(v: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Weight norm w = g * v / ||v||.

    LiteRT discussion, "Rewrites for the GPU": the positional conv carries a
    weight norm g*v/||v||.  Reading (the pages name no axis): one norm per
    kernel tap k, taken over all output and input channels of that tap, so
    g has one entry per tap.
    """
    norm = np.sqrt((v ** 2).sum(axis=(0, 1)))                            # [K]
    return v * (g.reshape(-1) / norm)[None, None, :]


def positional_conv(z: np.ndarray, w: np.ndarray, b: np.ndarray, groups: int) -> np.ndarray:
    """Grouped positional conv on z [B, T, d]; w [d, d/G, K] (already folded).

    p[b, t, o] = bias[o] + sum_k sum_i w[o, i, k] * zpad[b, t + k, g(o)*d/G + i]
    with zpad = z padded by K//2 zero frames on both sides.  Reading for even
    K (the pages are silent): the padded conv yields T + 1 frames and the
    last one is dropped, so frame t sees z[t - K/2 .. t + K/2 - 1].
    """
    bsz, t_len, d = z.shape
    c_out, cg, kernel = w.shape
    assert c_out == d and cg * groups == d
    pad = kernel // 2
    zp = np.zeros((bsz, t_len + 2 * pad, d), dtype=z.dtype)
    zp[:, pad:pad + t_len] = z
    t_full = t_len + 2 * pad - kernel + 1
    zg = zp.reshape(bsz, t_len + 2 * pad, groups, cg).transpose(2, 0, 1, 3)  # [G, B, Tp, Cg]
    wg = w.reshape(groups, cg, cg, kernel)                                  # [G, o, i, K]
    p = np.zeros((groups, bsz, t_full, cg), dtype=z.dtype)
    for k in range(kernel):
        a = zg[:, :, k:k + t_full, :].reshape(groups, bsz * t_full, cg)
        wk = np.ascontiguousarray(wg[:, :, :, k].transpose(0, 2, 1))     # [G, i, o]
        p += np.matmul(np.ascontiguousarray(a), wk).reshape(groups, bsz, t_full, cg)
    p = p.transpose(1, 2, 0, 3).reshape(bsz, t_full, d)
    if kernel % 2 == 0:
        p = p[:, :t_len]
    return p + b[None, None, :]


# ----------------------------------------------------------------------------
# transformer pieces
# ----------------------------------------------------------------------------
def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """softmax(s)_j = exp(s_j) / sum exp(s); the row max is subtracted first,
    which leaves the value unchanged."""
    m = s.max(axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=axis, keepdims=True)


# The projections that the FP8 mode quantizes (TensorRT README, "Recipe that
# was measured": q_proj, k_proj, v_proj, out_proj, intermediate_dense and
# output_dense of every encoder layer), keyed by the name of the tensor their
# input amax is stored under: q, k and v read the same input, so they share
# one activation amax.
FP8_INPUTS = ("attn.qkv", "attn.out", "ffn.fc1", "ffn.fc2")


def amax_key(layer: int, which: str) -> str:
    """Weight-table name of the calibrated input amax of projection `which`
    (one of FP8_INPUTS) of layer `layer`."""
    return f"layer{layer}.{which}.input_amax"


def linear(x: np.ndarray, W: dict, name: str, s_x: float | None = None) -> np.ndarray:
    """x W^T + b for the linear `name`.

    With s_x (FP8 mode) the input and the weight pass through e4m3
    quantize -> dequantize first, with the static per-tensor activation scale
    s_x and the per-tensor weight scale s_w = amax(|W|) / 448 (TensorRT README,
    "Recipe that was measured": input -> Quantize -> Dequantize -> MatMul <-
    Dequantize <- FP8 weight).  Dequantization is taken as exact scaling, so
    the product is (Q(x / s_x) Q(W / s_w)^T) s_x s_w.
    """
    dt = x.dtype
    w = W[name + ".weight"].astype(dt)
    if s_x is not None:
        s_w = np.abs(w).max() / E4M3_MAX
        x = quantize_e4m3(x / s_x) * s_x
        w = quantize_e4m3(w / s_w) * s_w
    return np.matmul(x, w.T) + W[name + ".bias"].astype(dt)


def _record(record: dict | None, key: str, x: np.ndarray) -> None:
    if record is not None:
        record[key] = max(record.get(key, 0.0), float(np.abs(x).max()))


def _act_scale(W: dict, fp8: bool, layer: int, which: str) -> float | None:
    return float(np.asarray(W[amax_key(layer, which)]).reshape(-1)[0]) / E4M3_MAX if fp8 else None


def self_attention(h: np.ndarray, W: dict, prefix: str, heads: int, fp8: bool = False,
                   record: dict | None = None, layer: int = 0) -> np.ndarray:
    """Multi-head self-attention over all T frames, no mask.

    LiteRT discussion, "Rewrites for the GPU": the bidirectional mask is
    removed, so attention is plain scaled dot-product attention over the
    whole window (short clips are zero-padded).  q/k/v/out projections carry
    biases (TensorRT README, "Recipe that was measured", lists q_proj,
    k_proj, v_proj, out_proj).  Scale 1/sqrt(d_head).  fp8: the four
    projections are FP8 (see linear); the attention matmuls and softmax are
    not.  record: receives the max |input| of the q/k/v and out projections
    (the calibration statistic of the FP8 recipe).
    """
    bsz, t_len, d = h.shape
    dh = d // heads
    dt = h.dtype
    _record(record, amax_key(layer, "attn.qkv"), h)
    sx = _act_scale(W, fp8, layer, "attn.qkv")
    q = linear(h, W, prefix + "q", sx).reshape(bsz, t_len, heads, dh).transpose(0, 2, 1, 3)
    k = linear(h, W, prefix + "k", sx).reshape(bsz, t_len, heads, dh).transpose(0, 2, 1, 3)
    v = linear(h, W, prefix + "v", sx).reshape(bsz, t_len, heads, dh).transpose(0, 2, 1, 3)
    s = np.matmul(q, k.transpose(0, 1, 3, 2)) / np.sqrt(dt.type(dh))   # [B, H, T, T]
    o = np.matmul(softmax(s, axis=-1), v)                               # [B, H, T, dh]
    o = o.transpose(0, 2, 1, 3).reshape(bsz, t_len, d)
    _record(record, amax_key(layer, "attn.out"), o)
    return linear(o, W, prefix + "out", _act_scale(W, fp8, layer, "attn.out"))


def feed_forward(h: np.ndarray, W: dict, prefix: str, act=None, fp8: bool = False,
                 record: dict | None = None, layer: int = 0) -> np.ndarray:
    """fc2(GELU(fc1(h))), both linears with bias (TensorRT README, "Recipe that
    was measured": intermediate_dense and output_dense); fp8 / record as in
    self_attention."""
    act = gelu if act is None else act
    _record(record, amax_key(layer, "ffn.fc1"), h)
    u = act(linear(h, W, prefix + "fc1", _act_scale(W, fp8, layer, "ffn.fc1")))
    _record(record, amax_key(layer, "ffn.fc2"), u)
    return linear(u, W, prefix + "fc2", _act_scale(W, fp8, layer, "ffn.fc2"))


# ----------------------------------------------------------------------------
# network
# ----------------------------------------------------------------------------
def num_frames(cfg, samples: int) -> int:
    """Output frames of the conv feature encoder for ``samples`` input
    samples: the unpadded conv length rule applied layer by layer."""
    n = int(samples)
    for k, s in zip(cfg.conv_kernel, cfg.conv_stride):
        n = conv_out_len(n, k, s)
    return n


def feature_encoder(cfg, W: dict, pcm: np.ndarray, valid: np.ndarray,
                    dtype=np.float64) -> np.ndarray:
    """Conv feature encoder: PCM [B, L] -> features [B, C, T].

    * Samples at or after valid[b] are taken as exact zeros, whatever the
      buffer holds (LiteRT discussion, "Rewrites for the GPU": short clips
      are zero-padded to the fixed window).
    * Group-norm variant: conv0 -> GroupNorm over time -> GELU, then
      conv_i -> GELU.  Layer-norm variant: every conv_i -> LayerNorm over the
      channels of each frame -> GELU.  Conv bias only where the config has it
      (TensorRT README, "Wav2Vec2 CTC layouts": group-normalized and per-frame
      layer-normalized feature encoders, with or without convolution bias).
    """
    dt = np.dtype(dtype)
    act = activation(cfg)
    x = np.asarray(pcm, dtype=dt).copy()
    for b in range(x.shape[0]):
        x[b, int(valid[b]):] = 0.0
    h = x[:, None, :]
    for i in range(len(cfg.conv_dim)):
        wk = W[f"fe.conv{i}.weight"].astype(dt)
        bk = W[f"fe.conv{i}.bias"].astype(dt) if cfg.conv_bias else None
        h = conv1d(h, wk, bk, cfg.conv_stride[i])
        if cfg.feat_norm == "layer":
            h = layer_norm(h, W[f"fe.norm{i}.weight"].astype(dt), W[f"fe.norm{i}.bias"].astype(dt),
                           cfg.eps, axis=1)
        elif i == 0:
            h = group_norm_over_time(h, W["fe.norm0.weight"].astype(dt), W["fe.norm0.bias"].astype(dt),
                                     cfg.eps)
        h = act(h)
    return h


def encoder(cfg, W: dict, feats: np.ndarray, fp8: bool = False, record: dict | None = None) -> np.ndarray:
    """Feature projection, positional conv and the transformer blocks.

    feats [B, C, T] -> hidden [B, T, d].

    * GELU is the exact erf form unless the config selects the tanh
      approximation (compatibility with the tanh-GELU export of the LiteRT
      discussion, "Rewrites for the GPU").
    * Feature projection: LayerNorm over C per frame, then Linear C -> d.
    * Positional conv: h = z + GELU(posconv(z)), with the weight norm folded
      from (v, g) on every call (LiteRT discussion, "Rewrites for the GPU").
    * Post-norm blocks (TensorRT README, "Wav2Vec2 CTC layouts": blocks keep
      the checkpoint's post-norm or stable pre-norm order; stable checkpoints
      apply the encoder-level norm after the blocks; reading: the post-norm
      layout applies it before them):
        h = LN(h);  per block: h = LN(h + MHA(h)); h = LN(h + FFN(h)).
      Stable pre-norm:
        per block: h = h + MHA(LN(h)); h = h + FFN(LN(h));  then h = LN(h).
    * fp8: the FP8 mode of the TensorRT README's FP8 quantization study, with
      the static activation amax of every projection input taken from the
      weight table (amax_key); record: collects those amax values instead.
    """
    dt = feats.dtype
    eps = cfg.eps
    act = activation(cfg)

    def g(name):
        return W[name].astype(dt)

    f = feats.transpose(0, 2, 1)                                         # [B, T, C]
    f = layer_norm(f, g("fp.norm.weight"), g("fp.norm.bias"), eps)
    z = np.matmul(f, g("fp.proj.weight").T) + g("fp.proj.bias")
    w_pos = fold_weight_norm(g("pos.weight_v"), g("pos.weight_g"))
    h = z + act(positional_conv(z, w_pos, g("pos.bias"), cfg.pos_groups))
    if not cfg.stable_layer_norm:
        h = layer_norm(h, g("enc.norm.weight"), g("enc.norm.bias"), eps)
    for l in range(cfg.layers):
        p = f"layer{l}."
        kw = dict(fp8=fp8, record=record, layer=l)
        if cfg.stable_layer_norm:
            a = layer_norm(h, g(p + "attn_norm.weight"), g(p + "attn_norm.bias"), eps)
            h = h + self_attention(a, W, p + "attn.", cfg.heads, **kw)
            a = layer_norm(h, g(p + "ffn_norm.weight"), g(p + "ffn_norm.bias"), eps)
            h = h + feed_forward(a, W, p + "ffn.", act, **kw)
        else:
            h = layer_norm(h + self_attention(h, W, p + "attn.", cfg.heads, **kw),
                           g(p + "attn_norm.weight"), g(p + "attn_norm.bias"), eps)
            h = layer_norm(h + feed_forward(h, W, p + "ffn.", act, **kw),
                           g(p + "ffn_norm.weight"), g(p + "ffn_norm.bias"), eps)
    if cfg.stable_layer_norm:
        h = layer_norm(h, g("enc.norm.weight"), g("enc.norm.bias"), eps)
    return h


def ctc_head(W: dict, h: np.ndarray) -> np.ndarray:
    """CTC logits = h W^T + b over the vocabulary (TensorRT README, "Recipe
    that was measured": the CTC head)."""
    dt = h.dtype
    return np.matmul(h, W["head.weight"].astype(dt).T) + W["head.bias"].astype(dt)


def valid_frames(cfg, valid: np.ndarray) -> np.ndarray:
    """Frames per row computed from valid samples only (LiteRT discussion,
    "Rewrites for the GPU": decoding runs over the valid frames)."""
    return np.array([num_frames(cfg, int(v)) for v in valid], dtype=np.int32)


def forward(cfg, W: dict, pcm: np.ndarray, valid: np.ndarray, dtype=np.float64, fp8: bool = False):
    """Whole network: (logits [B, T, V] in ``dtype``, valid frames int32 [B]).

    Logits are produced for every frame of the window; only the first
    valid-frames of each row are decoded.  fp8: the encoder projections in
    FP8 (encoder), with the input amax entries of W.
    """
    feats = feature_encoder(cfg, W, pcm, valid, dtype)
    h = encoder(cfg, W, feats, fp8=fp8)
    return ctc_head(W, h), valid_frames(cfg, valid)


def calibrate_amax(cfg, W: dict, pcm: np.ndarray, valid: np.ndarray, dtype=np.float64) -> dict:
    """Static activation calibration of the FP8 recipe (TensorRT README,
    "Recipe that was measured": max(abs(input)) of every quantized projection,
    recorded with forward pre-hooks on the float model over calibration
    clips): runs the float network on the given windows and returns
    {amax_key(l, which): float32 [1]} for every layer and FP8_INPUTS entry."""
    rec: dict = {}
    feats = feature_encoder(cfg, W, pcm, valid, dtype)
    encoder(cfg, W, feats, record=rec)
    return {k: np.array([v], np.float32) for k, v in rec.items()}


def forward_true_length(cfg, W: dict, pcm: np.ndarray, valid: np.ndarray, dtype=np.float64):
    """Every row run as its own true-length clip: (logits [B, T, V], frames [B]).

    Row b is the whole network applied to its first valid[b] samples alone,
    as one clip of exactly that length (TensorRT README, "Wav2Vec2 CTC
    layouts": the input is true-length PCM and no padded-batch attention mask
    is introduced).  So the conv layers, the group norm over time, the
    positional conv's zero padding and the attention of row b see only that
    clip.  Results sit on the frame grid of the full window (T = frames of
    pcm.shape[1] samples); frames at or after the row's own frame count are 0.
    """
    B, L = pcm.shape
    T = num_frames(cfg, L)
    out = np.zeros((B, T, cfg.vocab), dtype=np.dtype(dtype))
    vf = np.zeros(B, np.int32)
    for b in range(B):
        v = int(min(max(int(valid[b]), 0), L))
        n = num_frames(cfg, v)
        vf[b] = n
        if n == 0:
            continue
        logits, _ = forward(cfg, W, pcm[b:b + 1, :v], np.array([v], np.int32), dtype)
        out[b, :n] = logits[0]
    return out, vf


# ----------------------------------------------------------------------------
# greedy CTC decoding
# ----------------------------------------------------------------------------
def frame_argmax(logits: np.ndarray) -> np.ndarray:
    """Per-frame argmax over the vocabulary, lowest index on ties (the
    per-frame argmax of LiteRT discussion "fp16 / int8" and TensorRT README
    "Method").  int32 [..., T]."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def ctc_collapse(path, blank: int) -> np.ndarray:
    """Greedy (best-path) CTC collapse: merge runs of equal ids, then remove
    the blank id.  Textbook CTC decoding rule (Graves et al., 2006)."""
    out = []
    prev = None
    for a in path:
        a = int(a)
        if a != prev and a != blank:
            out.append(a)
        prev = a
    return np.array(out, dtype=np.int32)


def greedy_decode(logits: np.ndarray, vframes: np.ndarray, blank: int) -> list[np.ndarray]:
    """Token ids per row: argmax over the valid frames, then collapse."""
    a = frame_argmax(logits)
    return [ctc_collapse(a[b, :int(vframes[b])], blank) for b in range(a.shape[0])]
