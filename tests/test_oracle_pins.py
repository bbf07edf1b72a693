"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a closed form, a brute-force
loop written independently here, an invariant the mathematics fixes, a
library routine that computes the same special case, or (for the whole
network) an independent library implementation of Wav2Vec2ForCTC.  The
mutation tests at the end plant plausible mistakes into the oracle (on the
CPU) and show that the pins catch them.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def _tiny(**kw):
    return synth.TINY_1S_B1.replace(**kw)


# ----------------------------------------------------------------------------
# frame counts
# ----------------------------------------------------------------------------
def test_frame_counts_golden():
    cfg = synth.BASE_16S_B8
    for row in _read_golden("frame_counts.txt"):
        n, t = map(int, row.split())
        assert oracle.num_frames(cfg, n) == t, (n, t)


def test_frame_count_closed_form_all_lengths():
    """The layer-by-layer rule equals floor((L - 400) / 320) + 1 (0 below 400)."""
    cfg = synth.BASE_16S_B8
    for n in list(range(0, 5000)) + list(range(5000, 400000, 37)):
        want = 0 if n < 400 else (n - 400) // 320 + 1
        assert oracle.num_frames(cfg, n) == want, n


@pytest.mark.parametrize("cfg", [synth.TINY_1S_B1, _tiny(window=16000 + 333)])
def test_feature_encoder_length_matches_frame_count(cfg):
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    feats = oracle.feature_encoder(cfg, W, pcm, valid)
    assert feats.shape == (cfg.batch, cfg.conv_dim[-1], oracle.num_frames(cfg, cfg.window))


# ----------------------------------------------------------------------------
# convolutions
# ----------------------------------------------------------------------------
def _conv_loops(x, w, b, s):
    B, C, L = x.shape
    O, _, K = w.shape
    T = (L - K) // s + 1
    y = np.zeros((B, O, T))
    for bb in range(B):
        for o in range(O):
            for t in range(T):
                acc = 0.0 if b is None else b[o]
                for c in range(C):
                    for k in range(K):
                        acc += w[o, c, k] * x[bb, c, s * t + k]
                y[bb, o, t] = acc
    return y


@pytest.mark.parametrize("K,s,C,O,L", [(3, 2, 3, 4, 17), (2, 2, 2, 3, 10), (10, 5, 1, 4, 57), (1, 1, 2, 2, 5)])
@pytest.mark.parametrize("bias", [False, True])
def test_conv1d_bruteforce(K, s, C, O, L, bias):
    rng = np.random.default_rng(K * 100 + L)
    x = rng.standard_normal((2, C, L))
    w = rng.standard_normal((O, C, K))
    b = rng.standard_normal(O) if bias else None
    np.testing.assert_allclose(oracle.conv1d(x, w, b, s), _conv_loops(x, w, b, s), rtol=0, atol=1e-12)


def test_conv0_vs_numpy_convolve():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 1, 1003))
    w = rng.standard_normal((6, 1, 10))
    y = oracle.conv1d(x, w, None, 5)
    for o in range(6):
        ref = np.convolve(x[0, 0], w[o, 0, ::-1], mode="valid")[::5]
        np.testing.assert_allclose(y[0, o], ref, rtol=0, atol=1e-12)


def test_conv_k2_s2_is_reshape_matmul():
    """With kernel = stride = 2 the conv is a plain matmul over frame pairs."""
    rng = np.random.default_rng(6)
    B, C, O, T = 2, 5, 7, 9
    x = rng.standard_normal((B, C, 2 * T + 1))          # odd length: last sample unused
    w = rng.standard_normal((O, C, 2))
    pairs = x[:, :, :2 * T].reshape(B, C, T, 2).transpose(0, 2, 3, 1).reshape(B, T, 2 * C)
    wm = w.transpose(0, 2, 1).reshape(O, 2 * C)
    ref = (pairs @ wm.T).transpose(0, 2, 1)
    np.testing.assert_allclose(oracle.conv1d(x, w, None, 2), ref, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# norms and GELU
# ----------------------------------------------------------------------------
def test_group_norm_invariants():
    rng = np.random.default_rng(7)
    y = rng.standard_normal((3, 4, 257)) * rng.uniform(0.1, 3, (3, 4, 1)) + rng.standard_normal((3, 4, 1))
    eps = 1e-5
    out = oracle.group_norm_over_time(y, np.ones(4), np.zeros(4), eps)
    var_in = y.var(axis=2)
    np.testing.assert_allclose(out.mean(axis=2), 0, atol=1e-12)
    np.testing.assert_allclose(out.var(axis=2), var_in / (var_in + eps), rtol=1e-12)
    g, b = rng.standard_normal(4), rng.standard_normal(4)
    out2 = oracle.group_norm_over_time(y, g, b, eps)
    np.testing.assert_allclose(out2, out * g[None, :, None] + b[None, :, None], atol=1e-12)


def test_group_norm_matches_torch_groupnorm():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    y = rng.standard_normal((2, 6, 101))
    g, b = rng.standard_normal(6), rng.standard_normal(6)
    gn = torch.nn.GroupNorm(6, 6, eps=1e-5).double()
    with torch.no_grad():
        gn.weight.copy_(torch.from_numpy(g))
        gn.bias.copy_(torch.from_numpy(b))
        ref = gn(torch.from_numpy(y)).numpy()
    np.testing.assert_allclose(oracle.group_norm_over_time(y, g, b, 1e-5), ref, atol=1e-12)


def test_layer_norm_invariants():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 33)) * 2.5 + 1.0
    eps = 1e-5
    out = oracle.layer_norm(x, np.ones(33), np.zeros(33), eps)
    var_in = x.var(axis=1)
    np.testing.assert_allclose(out.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(out.var(axis=1), var_in / (var_in + eps), rtol=1e-12)
    # channel axis form used by the layer-norm feature encoder
    y = rng.standard_normal((2, 7, 11))
    g, b = rng.standard_normal(7), rng.standard_normal(7)
    a1 = oracle.layer_norm(y, g, b, eps, axis=1)
    a2 = oracle.layer_norm(y.transpose(0, 2, 1), g, b, eps).transpose(0, 2, 1)
    np.testing.assert_allclose(a1, a2, atol=1e-12)


def test_gelu_vs_math_erf():
    xs = np.linspace(-8, 8, 1601)
    ref = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs])
    np.testing.assert_allclose(oracle.gelu(xs), ref, rtol=1e-14, atol=1e-15)
    assert oracle.gelu(np.array(0.0)) == 0.0
    np.testing.assert_allclose(oracle.gelu(xs) - oracle.gelu(-xs), xs, atol=1e-13)
    # Phi(1) = 0.8413447460685429... (standard normal CDF at 1)
    np.testing.assert_allclose(oracle.gelu(np.array(1.0)), 0.8413447460685429, rtol=1e-15)


def test_gelu_tanh_matches_torch_tanh_approximation():
    torch = pytest.importorskip("torch")
    xs = np.linspace(-10, 10, 2001)
    ref = torch.nn.functional.gelu(torch.from_numpy(xs), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(xs), ref, rtol=1e-13, atol=1e-15)
    assert oracle.gelu_tanh(np.array(0.0)) == 0.0
    # the approximation stays within 5e-4 of the exact form (Hendrycks & Gimpel)
    assert np.abs(oracle.gelu_tanh(xs) - oracle.gelu(xs)).max() < 5e-4


def test_activation_follows_config():
    assert oracle.activation(_tiny()) is oracle.gelu
    assert oracle.activation(_tiny(gelu="tanh")) is oracle.gelu_tanh


# ----------------------------------------------------------------------------
# weight norm and positional conv
# ----------------------------------------------------------------------------
def test_weight_norm_tap_norms_equal_gain():
    rng = np.random.default_rng(10)
    v = rng.standard_normal((8, 2, 6))
    g = rng.uniform(0.5, 2, 6)
    w = oracle.fold_weight_norm(v, g)
    np.testing.assert_allclose(np.sqrt((w ** 2).sum(axis=(0, 1))), g, rtol=1e-14)
    # direction unchanged
    np.testing.assert_allclose(w / np.linalg.norm(w[:, :, 0]) * np.linalg.norm(v[:, :, 0]), w / g[0] * np.linalg.norm(v[:, :, 0]), rtol=1e-14)


def test_weight_norm_matches_torch_parametrization():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    conv = torch.nn.Conv1d(8, 8, 6, groups=4).double()
    conv = torch.nn.utils.parametrizations.weight_norm(conv, name="weight", dim=2)
    v = rng.standard_normal((8, 2, 6))
    g = rng.uniform(0.5, 2, 6)
    with torch.no_grad():
        conv.parametrizations.weight.original0.copy_(torch.from_numpy(g.reshape(1, 1, 6)))
        conv.parametrizations.weight.original1.copy_(torch.from_numpy(v))
        ref = conv.weight.numpy()
    np.testing.assert_allclose(oracle.fold_weight_norm(v, g), ref, rtol=1e-13)


def _pos_conv_loops(z, w, b, G):
    B, T, d = z.shape
    _, cg, K = w.shape
    pad = K // 2
    out = np.zeros((B, T, d))
    for bb in range(B):
        for t in range(T):
            for o in range(d):
                g = o // cg
                acc = b[o]
                for k in range(K):
                    src = t - pad + k
                    if 0 <= src < T:
                        for i in range(cg):
                            acc += w[o, i, k] * z[bb, src, g * cg + i]
                out[bb, t, o] = acc
    return out


@pytest.mark.parametrize("K", [4, 5, 16])
def test_positional_conv_bruteforce(K):
    rng = np.random.default_rng(12 + K)
    B, T, d, G = 2, 7, 6, 3
    z = rng.standard_normal((B, T, d))
    w = rng.standard_normal((d, d // G, K))
    b = rng.standard_normal(d)
    np.testing.assert_allclose(oracle.positional_conv(z, w, b, G), _pos_conv_loops(z, w, b, G), atol=1e-12)


def test_positional_conv_matches_torch_conv_drop_last():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    B, T, d, G, K = 2, 20, 8, 4, 6
    z = rng.standard_normal((B, T, d))
    w = rng.standard_normal((d, d // G, K))
    b = rng.standard_normal(d)
    ref = torch.nn.functional.conv1d(torch.from_numpy(z).transpose(1, 2), torch.from_numpy(w),
                                     torch.from_numpy(b), padding=K // 2, groups=G)
    ref = ref[:, :, :-1].transpose(1, 2).numpy()
    np.testing.assert_allclose(oracle.positional_conv(z, w, b, G), ref, atol=1e-12)


# ----------------------------------------------------------------------------
# attention, feed-forward
# ----------------------------------------------------------------------------
def _attn_weights(rng, d):
    W = {}
    for p in ("q", "k", "v", "out"):
        W[f"a.{p}.weight"] = rng.standard_normal((d, d))
        W[f"a.{p}.bias"] = rng.standard_normal(d)
    return W


def _attn_loops(h, W, heads):
    B, T, d = h.shape
    dh = d // heads

    def lin(name, x):
        Wm, bv = W[f"a.{name}.weight"], W[f"a.{name}.bias"]
        return np.array([[sum(Wm[o, i] * x[t, i] for i in range(d)) + bv[o] for o in range(d)] for t in range(x.shape[0])])

    out = np.zeros((B, T, d))
    for bb in range(B):
        q, k, v = lin("q", h[bb]), lin("k", h[bb]), lin("v", h[bb])
        o = np.zeros((T, d))
        for hh in range(heads):
            sl = slice(hh * dh, (hh + 1) * dh)
            for t in range(T):
                sc = [sum(q[t, sl][j] * k[u, sl][j] for j in range(dh)) / math.sqrt(dh) for u in range(T)]
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                z = sum(e)
                for j in range(dh):
                    o[t, hh * dh + j] = sum(e[u] / z * v[u, hh * dh + j] for u in range(T))
        out[bb] = lin("out", o)
    return out


@pytest.mark.parametrize("T,d,heads", [(1, 4, 1), (5, 4, 2), (8, 8, 2)])
def test_attention_bruteforce(T, d, heads):
    rng = np.random.default_rng(T * 10 + d)
    h = rng.standard_normal((2, T, d))
    W = _attn_weights(rng, d)
    np.testing.assert_allclose(oracle.self_attention(h, W, "a.", heads), _attn_loops(h, W, heads), atol=1e-11)


def test_attention_single_frame_returns_value_path():
    """With T = 1 the softmax is exactly 1, so MHA(h) = out(v(h))."""
    rng = np.random.default_rng(14)
    d = 6
    h = rng.standard_normal((3, 1, d))
    W = _attn_weights(rng, d)
    v = h @ W["a.v.weight"].T + W["a.v.bias"]
    ref = v @ W["a.out.weight"].T + W["a.out.bias"]
    np.testing.assert_allclose(oracle.self_attention(h, W, "a.", 2), ref, atol=1e-13)


def test_softmax_rows_sum_to_one_and_match_direct_form():
    rng = np.random.default_rng(15)
    s = rng.standard_normal((4, 9)) * 3
    p = oracle.softmax(s)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-15)
    direct = np.exp(s) / np.exp(s).sum(axis=-1, keepdims=True)
    np.testing.assert_allclose(p, direct, rtol=1e-14)


def test_feed_forward_bruteforce():
    rng = np.random.default_rng(16)
    d, F = 4, 6
    W = {"f.fc1.weight": rng.standard_normal((F, d)), "f.fc1.bias": rng.standard_normal(F),
         "f.fc2.weight": rng.standard_normal((d, F)), "f.fc2.bias": rng.standard_normal(d)}
    h = rng.standard_normal((2, 3, d))
    ref = np.zeros_like(h)
    for b in range(2):
        for t in range(3):
            u = [sum(W["f.fc1.weight"][j, i] * h[b, t, i] for i in range(d)) + W["f.fc1.bias"][j] for j in range(F)]
            g = [0.5 * x * (1 + math.erf(x / math.sqrt(2))) for x in u]
            for o in range(d):
                ref[b, t, o] = sum(W["f.fc2.weight"][o, j] * g[j] for j in range(F)) + W["f.fc2.bias"][o]
    np.testing.assert_allclose(oracle.feed_forward(h, W, "f."), ref, atol=1e-12)


# ----------------------------------------------------------------------------
# CTC decoding
# ----------------------------------------------------------------------------
def _parse(tok):
    tok = tok.strip()
    return [] if tok == "-" else [int(v) for v in tok.split()]


def test_ctc_collapse_golden():
    rows = _read_golden("ctc_collapse_cases.txt")
    assert len(rows) >= 10
    for row in rows:
        src, want = row.split("|")
        got = oracle.ctc_collapse(_parse(src), 0)
        assert got.tolist() == _parse(want), row


def test_greedy_decode_fake_engine():
    """One-hot logits built from a hand-written path decode to its collapse."""
    paths = [[0, 0, 5, 5, 0, 5, 7, 7, 0, 3], [1, 1, 1, 0, 2, 2, 9, 9, 9, 9], [0] * 10]
    vf = np.array([9, 10, 0], np.int32)
    V = 12
    logits = np.full((3, 10, V), -1.0)
    for b, p in enumerate(paths):
        for t, a in enumerate(p):
            logits[b, t, a] = 2.0
    ids = oracle.greedy_decode(logits, vf, 0)
    assert ids[0].tolist() == [5, 5, 7]
    assert ids[1].tolist() == [1, 2, 9]
    assert ids[2].tolist() == []


def test_argmax_lowest_index_on_ties():
    logits = np.array([[[1.0, 3.0, 3.0, 0.0], [0.0, 0.0, 0.0, 0.0], [2.0, 1.0, 2.0, 2.0]]])
    assert oracle.frame_argmax(logits).tolist() == [[1, 0, 0]]


# ----------------------------------------------------------------------------
# whole network
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("stable", [False, True])
def test_all_zero_pcm_gives_zero_logits(stable):
    """Zero PCM with zero biases and unit gains: every stage maps 0 to 0
    (GN/LN of a constant row is beta = 0, GELU(0) = 0, attention averages
    zero values), so logits are exactly 0 and nothing is decoded."""
    cfg = _tiny(rand_affine=False, stable_layer_norm=stable, feat_norm="layer" if stable else "group",
                conv_bias=stable, batch=2)
    W = synth.make_weights(cfg)
    pcm = np.zeros((2, cfg.window), np.float32)
    logits, vf = oracle.forward(cfg, W, pcm, np.array([cfg.window, 5000], np.int32))
    assert np.all(logits == 0.0)
    assert vf.tolist() == [49, 15]
    assert [x.tolist() for x in oracle.greedy_decode(logits, vf, 0)] == [[], []]


def test_batch_permutation_equivariance():
    cfg = _tiny(batch=3, valid_range=(6000, 16000))
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    lg, vf = oracle.forward(cfg, W, pcm, valid)
    perm = [2, 0, 1]
    lg2, vf2 = oracle.forward(cfg, W, pcm[perm], valid[perm])
    np.testing.assert_allclose(lg2, lg[perm], rtol=0, atol=1e-12)
    assert vf2.tolist() == vf[perm].tolist()


def test_samples_beyond_valid_are_ignored():
    cfg = _tiny(batch=2, valid_range=(5000, 12000))
    W = synth.make_weights(cfg)
    pcm0, valid = synth.make_pcm(cfg)
    pcm1, _ = synth.make_pcm(cfg, valid=valid, pad_garbage=True)
    assert not np.array_equal(pcm0, pcm1)
    a, _ = oracle.forward(cfg, W, pcm0, valid)
    b, _ = oracle.forward(cfg, W, pcm1, valid)
    assert np.array_equal(a, b)


def test_fp32_run_within_bound_of_fp64():
    cfg = synth.TINY_1S_B1
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    a, _ = oracle.forward(cfg, W, pcm, valid, dtype=np.float64)
    b, _ = oracle.forward(cfg, W, pcm, valid, dtype=np.float32)
    assert b.dtype == np.float32
    assert np.abs(a - b).max() < 1e-4


# ----------------------------------------------------------------------------
# independent implementation of the same network: transformers' Wav2Vec2ForCTC
# ----------------------------------------------------------------------------
def _hf_name(n):
    if n.startswith("fe.conv"):
        i, rest = n[len("fe.conv"):].split(".", 1)
        return f"wav2vec2.feature_extractor.conv_layers.{i}.conv.{rest}"
    if n.startswith("fe.norm"):
        i, rest = n[len("fe.norm"):].split(".", 1)
        return f"wav2vec2.feature_extractor.conv_layers.{i}.layer_norm.{rest}"
    fixed = {"fp.norm.weight": "wav2vec2.feature_projection.layer_norm.weight",
             "fp.norm.bias": "wav2vec2.feature_projection.layer_norm.bias",
             "fp.proj.weight": "wav2vec2.feature_projection.projection.weight",
             "fp.proj.bias": "wav2vec2.feature_projection.projection.bias",
             "pos.weight_v": "wav2vec2.encoder.pos_conv_embed.conv.parametrizations.weight.original1",
             "pos.weight_g": "wav2vec2.encoder.pos_conv_embed.conv.parametrizations.weight.original0",
             "pos.bias": "wav2vec2.encoder.pos_conv_embed.conv.bias",
             "enc.norm.weight": "wav2vec2.encoder.layer_norm.weight",
             "enc.norm.bias": "wav2vec2.encoder.layer_norm.bias",
             "head.weight": "lm_head.weight", "head.bias": "lm_head.bias"}
    if n in fixed:
        return fixed[n]
    l, rest = n[len("layer"):].split(".", 1)
    sub = {"attn.q": "attention.q_proj", "attn.k": "attention.k_proj", "attn.v": "attention.v_proj",
           "attn.out": "attention.out_proj", "attn_norm": "layer_norm", "ffn.fc1": "feed_forward.intermediate_dense",
           "ffn.fc2": "feed_forward.output_dense", "ffn_norm": "final_layer_norm"}
    head, leaf = rest.rsplit(".", 1)
    return f"wav2vec2.encoder.layers.{l}.{sub[head]}.{leaf}"


def _hf_model(cfg, W):
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers")
    hc = tr.Wav2Vec2Config(
        vocab_size=cfg.vocab, hidden_size=cfg.hidden, num_hidden_layers=cfg.layers,
        num_attention_heads=cfg.heads, intermediate_size=cfg.ffn, conv_dim=cfg.conv_dim,
        conv_kernel=cfg.conv_kernel, conv_stride=cfg.conv_stride, conv_bias=cfg.conv_bias,
        num_conv_pos_embeddings=cfg.pos_kernel, num_conv_pos_embedding_groups=cfg.pos_groups,
        feat_extract_norm=cfg.feat_norm, do_stable_layer_norm=cfg.stable_layer_norm,
        hidden_act="gelu_new" if cfg.gelu == "tanh" else "gelu",
        feat_extract_activation="gelu_new" if cfg.gelu == "tanh" else "gelu", layer_norm_eps=cfg.eps,
        pad_token_id=cfg.blank_id)
    torch.manual_seed(0)
    model = tr.Wav2Vec2ForCTC(hc).double().eval()
    sd = model.state_dict()
    new = {}
    for n, a in W.items():
        key = _hf_name(n)
        assert key in sd, key
        new[key] = torch.from_numpy(a.astype(np.float64)).reshape(sd[key].shape)
    missing = set(sd) - set(new) - {"wav2vec2.masked_spec_embed"}
    assert not missing, missing
    model.load_state_dict(new, strict=False)
    return model


def _hf_logits(cfg, W, pcm, model=None):
    import torch
    model = model if model is not None else _hf_model(cfg, {k: v for k, v in W.items() if "amax" not in k})
    with torch.no_grad():
        return model(torch.from_numpy(pcm.astype(np.float64))).logits.numpy()


_VARIANTS = {
    "group_postnorm": dict(),
    "layer_stable": dict(feat_norm="layer", conv_bias=True, stable_layer_norm=True),
    "group_postnorm_odd_pos_kernel": dict(pos_kernel=15),
    "layer_stable_tanh_gelu": dict(feat_norm="layer", conv_bias=True, stable_layer_norm=True, gelu="tanh"),
}


@pytest.mark.slow
@pytest.mark.parametrize("variant", sorted(_VARIANTS))
def test_whole_network_matches_transformers_wav2vec2forctc(variant):
    cfg = _tiny(batch=2, **_VARIANTS[variant])
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    ours, _ = oracle.forward(cfg, W, pcm, valid)
    ref = _hf_logits(cfg, W, pcm)
    assert ours.shape == ref.shape
    assert np.abs(ours - ref).max() < 1e-10


# ----------------------------------------------------------------------------
# true-length mode: every row is its own unpadded clip
# ----------------------------------------------------------------------------
@pytest.mark.slow
@pytest.mark.parametrize("variant", ["group_postnorm", "layer_stable"])
def test_true_length_rows_match_transformers_on_the_unpadded_clip(variant):
    # rows of different true lengths, one of them the whole window
    cfg = _tiny(batch=3, **_VARIANTS[variant])
    W = synth.make_weights(cfg)
    valid = np.array([cfg.window, 9321, 4410], np.int32)
    pcm, _ = synth.make_pcm(cfg, valid=valid, pad_garbage=True)
    ours, vf = oracle.forward_true_length(cfg, W, pcm, valid)
    T = oracle.num_frames(cfg, cfg.window)
    assert ours.shape == (3, T, cfg.vocab)
    for b in range(3):
        n = oracle.num_frames(cfg, int(valid[b]))
        assert vf[b] == n
        ref = _hf_logits(cfg, W, pcm[b:b + 1, :valid[b]])[0]
        assert ref.shape == (n, cfg.vocab)
        assert np.abs(ours[b, :n] - ref).max() < 1e-10
        assert not ours[b, n:].any()


def test_true_length_full_rows_equal_the_padded_window():
    cfg = _tiny(batch=2)
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg, valid=np.array([cfg.window, cfg.window], np.int32))
    a, va = oracle.forward_true_length(cfg, W, pcm, valid)
    b, vb = oracle.forward(cfg, W, pcm, valid)
    assert np.array_equal(va, vb)
    assert np.array_equal(a, b)


def test_true_length_rows_are_independent_and_differ_from_padded_mode():
    cfg = _tiny(batch=2)
    W = synth.make_weights(cfg)
    valid = np.array([7000, 12000], np.int32)
    pcm, _ = synth.make_pcm(cfg, valid=valid)
    a, _ = oracle.forward_true_length(cfg, W, pcm, valid)
    pcm2 = pcm.copy()
    pcm2[1] = synth.make_pcm(cfg, seed=999, valid=valid)[0][1]
    valid2 = valid.copy()
    valid2[1] = 15000
    b, _ = oracle.forward_true_length(cfg, W, pcm2, valid2)
    assert np.array_equal(a[0], b[0])
    # the padded window (group norm over the zero tail, attention over every
    # frame) is a different computation for a short row
    p, _ = oracle.forward(cfg, W, pcm, valid)
    n = oracle.num_frames(cfg, 7000)
    assert np.abs(p[0, :n] - a[0, :n]).max() > 1e-4


def test_true_length_short_rows():
    cfg = _tiny(batch=3)
    W = synth.make_weights(cfg)
    valid = np.array([0, 399, 400], np.int32)
    pcm, _ = synth.make_pcm(cfg, valid=valid)
    out, vf = oracle.forward_true_length(cfg, W, pcm, valid)
    assert vf.tolist() == [0, 0, 1]
    assert not out[0].any() and not out[1].any()
    assert not out[2, 1:].any() and np.abs(out[2, 0]).max() > 0


# ----------------------------------------------------------------------------
# mutation tests: plant a mistake in the oracle and show a pin catches it
# ----------------------------------------------------------------------------
def _tanh_gelu(x):
    return 0.5 * x * (1 + np.tanh(np.sqrt(2 / np.pi) * (x + 0.044715 * x ** 3)))


@pytest.mark.slow
@pytest.mark.parametrize("mutation", ["tanh_gelu", "pos_conv_keeps_first_drop", "ln_without_eps",
                                      "no_valid_mask", "attention_scale_dh"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    from oracle import w2v2_oracle as m
    cfg = _tiny(batch=2, valid_range=(9000, 16000))
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    pcm_hf = pcm.copy()
    good, _ = m.forward(cfg, W, pcm, valid)
    if mutation == "tanh_gelu":
        monkeypatch.setattr(m, "gelu", _tanh_gelu)
    elif mutation == "pos_conv_keeps_first_drop":
        orig = m.positional_conv

        def shifted(z, w, b, groups):
            zp = np.concatenate([z[:, 1:], np.zeros_like(z[:, :1])], axis=1)
            return orig(zp, w, b, groups)
        monkeypatch.setattr(m, "positional_conv", shifted)
    elif mutation == "ln_without_eps":
        orig_ln = m.layer_norm
        monkeypatch.setattr(m, "layer_norm", lambda x, g, b, eps, axis=-1: orig_ln(x, g, b, 0.0, axis))
    elif mutation == "no_valid_mask":
        pcm = synth.make_pcm(cfg, valid=valid, pad_garbage=True)[0]
        good, _ = oracle.forward(cfg, W, pcm, valid)
        # the planted mistake: forget to zero past the valid length
        bad, _ = oracle.forward(cfg, W, pcm, np.full_like(valid, cfg.window))
        assert np.abs(bad - good).max() > 1e-6
        return
    elif mutation == "attention_scale_dh":
        dh = cfg.hidden // cfg.heads  # planted: scale 1/d_head instead of 1/sqrt(d_head)
        monkeypatch.setattr(m, "softmax", lambda s, axis=-1: oracle.softmax(s / np.sqrt(dh), axis))
    bad, _ = m.forward(cfg, W, pcm, valid)
    monkeypatch.undo()
    ref = _hf_logits(cfg, W, pcm_hf * (np.arange(cfg.window)[None, :] < valid[:, None]))
    # the pin's tolerance is 1e-10; a planted mistake must move the logits
    # far outside it
    assert np.abs(good - ref).max() < 1e-10
    assert np.abs(bad - ref).max() > 1e-8


# ----------------------------------------------------------------------------
# FP8 (e4m3) projections: quantizer, calibration, quantized network
# ----------------------------------------------------------------------------
def _torch_e4m3(x):
    """torch's own float8_e4m3fn cast (round to nearest even), with the
    saturation of the recipe applied first as a clamp."""
    torch = pytest.importorskip("torch")
    t = torch.from_numpy(np.clip(np.asarray(x, np.float64), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_quantize_e4m3_matches_torch_float8_cast():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-14, 7, 200000))
    x = x[np.abs(x) <= 448]
    assert np.array_equal(oracle.quantize_e4m3(x), _torch_e4m3(x))


def _ties_go_to_even(qfun):
    """Midpoints of neighbouring e4m3 values quantize to the neighbour whose
    code (torch's bit pattern) is even, symmetrically in sign."""
    torch = pytest.importorskip("torch")
    vals = torch.arange(127, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    pos = np.unique(vals)
    mids = (pos[:-1] + pos[1:]) / 2
    got = qfun(mids)
    code_of = {float(v): int(c) for c, v in enumerate(vals)}
    ok = all(g in (lo, hi) and code_of[float(g)] % 2 == 0 for lo, hi, g in zip(pos[:-1], pos[1:], got))
    return ok and np.array_equal(qfun(-mids), -got)


def test_quantize_e4m3_grid_ties_and_saturation():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    vals = codes.to(torch.float64).numpy()
    finite = np.isfinite(vals)
    assert finite.sum() == 254                      # 0x7f and 0xff are NaN
    grid = np.unique(vals[finite])
    assert len(grid) == 253 and grid.max() == 448 and np.min(grid[grid > 0]) == 2.0 ** -9
    # every grid value is a fixed point
    assert np.array_equal(oracle.quantize_e4m3(grid), grid)
    assert _ties_go_to_even(oracle.quantize_e4m3)
    # saturation instead of NaN beyond the largest value
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf])
    assert np.all(oracle.quantize_e4m3(big) == 448.0)
    assert np.all(oracle.quantize_e4m3(-big) == -448.0)


def _hf_amax_hooks(model, layers):
    rec = {}

    def hook(key):
        def f(mod, args):
            rec[key] = max(rec.get(key, 0.0), float(args[0].abs().max()))
        return f
    hs = []
    for l, layer in enumerate(model.wav2vec2.encoder.layers[:layers]):
        hs.append(layer.attention.q_proj.register_forward_pre_hook(hook(oracle.amax_key(l, "attn.qkv"))))
        hs.append(layer.attention.out_proj.register_forward_pre_hook(hook(oracle.amax_key(l, "attn.out"))))
        hs.append(layer.feed_forward.intermediate_dense.register_forward_pre_hook(hook(oracle.amax_key(l, "ffn.fc1"))))
        hs.append(layer.feed_forward.output_dense.register_forward_pre_hook(hook(oracle.amax_key(l, "ffn.fc2"))))
    return rec, hs


@pytest.mark.slow
@pytest.mark.parametrize("variant", ["group_postnorm", "layer_stable"])
def test_calibrate_amax_matches_transformers_pre_hooks(variant):
    cfg = _tiny(batch=2, **_VARIANTS[variant])
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    amax = oracle.calibrate_amax(cfg, W, pcm, valid)
    assert sorted(amax) == sorted(oracle.amax_key(l, w) for l in range(cfg.layers) for w in oracle.FP8_INPUTS)
    model = _hf_model(cfg, W)
    rec, hs = _hf_amax_hooks(model, cfg.layers)
    _hf_logits(cfg, W, pcm, model)
    for h in hs:
        h.remove()
    for k, v in amax.items():
        assert abs(float(v[0]) - np.float32(rec[k])) == 0, (k, v, rec[k])


def _hf_fp8_logits(cfg, W, pcm):
    """transformers' network with the FP8 recipe applied through torch: the
    72-projection weights replaced by their e4m3 quantize-dequantize with
    per-tensor scale amax/448, the inputs of those projections passed through
    quantize-dequantize with the calibrated scales (forward pre-hooks)."""
    torch = pytest.importorskip("torch")
    model = _hf_model(cfg, {k: v for k, v in W.items() if "amax" not in k})
    hs = []
    for l, layer in enumerate(model.wav2vec2.encoder.layers):
        mods = {"attn.qkv": [layer.attention.q_proj, layer.attention.k_proj, layer.attention.v_proj],
                "attn.out": [layer.attention.out_proj], "ffn.fc1": [layer.feed_forward.intermediate_dense],
                "ffn.fc2": [layer.feed_forward.output_dense]}
        for which, ms in mods.items():
            s_x = float(W[oracle.amax_key(l, which)][0]) / 448.0
            for mod in ms:
                w = mod.weight.data.numpy()
                s_w = np.abs(w).max() / 448.0
                mod.weight.data = torch.from_numpy(_torch_e4m3(w / s_w) * s_w)

                def pre(m, args, s_x=s_x):
                    return (torch.from_numpy(_torch_e4m3(args[0].numpy() / s_x) * s_x),)
                hs.append(mod.register_forward_pre_hook(pre))
    return _hf_logits(cfg, W, pcm, model)


@pytest.mark.slow
@pytest.mark.parametrize("variant", ["group_postnorm", "layer_stable"])
def test_fp8_network_matches_transformers_with_torch_fake_quant(variant):
    cfg = _tiny(batch=2, **_VARIANTS[variant])
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    cal_pcm, cal_valid = synth.make_pcm(cfg, seed=cfg.pcm_seed + 50)
    # half the calibrated range, so that the test inputs also saturate
    amax = {k: v * np.float32(0.5) for k, v in oracle.calibrate_amax(cfg, W, cal_pcm, cal_valid).items()}
    W8 = dict(W, **amax)
    ours, _ = oracle.forward(cfg, W8, pcm, valid, fp8=True)
    ref = _hf_fp8_logits(cfg, W8, pcm * (np.arange(cfg.window)[None, :] < valid[:, None]))
    plain, _ = oracle.forward(cfg, W, pcm, valid)
    assert np.abs(ours - ref).max() < 1e-9
    # the quantization does move the logits
    assert np.abs(ours - plain).max() > 1e-3


@pytest.mark.slow
@pytest.mark.parametrize("mutation", ["per_channel_weight_scale", "round_half_up", "no_saturation"])
def test_fp8_planted_mistakes_are_caught(monkeypatch, mutation):
    from oracle import w2v2_oracle as m
    cfg = _tiny(batch=2)
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    cal_pcm, cal_valid = synth.make_pcm(cfg, seed=cfg.pcm_seed + 50)
    W8 = dict(W, **{k: v * np.float32(0.5) for k, v in oracle.calibrate_amax(cfg, W, cal_pcm, cal_valid).items()})
    q = m.quantize_e4m3
    if mutation == "per_channel_weight_scale":
        def lin(x, Wt, name, s_x=None):
            w = Wt[name + ".weight"].astype(x.dtype)
            if s_x is not None:
                s_w = np.abs(w).max(axis=1, keepdims=True) / 448.0
                x = q(x / s_x) * s_x
                w = q(w / s_w) * s_w
            return np.matmul(x, w.T) + Wt[name + ".bias"]
        monkeypatch.setattr(m, "linear", lin)
    elif mutation == "round_half_up":
        # ties essentially never occur in network data: the quantizer's own
        # tie pin is the one that catches this
        def qu(x):
            a = np.abs(np.asarray(x, np.float64))
            _, e = np.frexp(a)
            step = np.ldexp(1.0, np.clip(e - 1, -6, 8) - 3)
            return np.copysign(np.minimum(np.floor(a / step + 0.5) * step, 448.0), x)
        assert _ties_go_to_even(q) and not _ties_go_to_even(qu)
        return
    elif mutation == "no_saturation":
        monkeypatch.setattr(m, "quantize_e4m3", lambda x: np.where(np.abs(x) > 448, np.nan, q(x)))
    bad, _ = m.forward(cfg, W8, pcm, valid, fp8=True)
    monkeypatch.undo()
    ref = _hf_fp8_logits(cfg, W8, pcm * (np.arange(cfg.window)[None, :] < valid[:, None]))
    assert not (np.abs(bad - ref).max() < 1e-9)
