"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Gates (fixed by the workload definitions):
  * fp32 mode: max |logits - oracle| <= 1e-3 over every frame of the window.
  * fp16 mode (fp16 operands, fp32 accumulation / norms / softmax): Pearson
    correlation of the logits over the valid frames >= 0.999 and per-frame
    argmax agreement over the valid frames >= 99.5%.
  * CTC ids: bit-exact given the same per-frame argmax (the GPU collapse of
    the GPU argmax equals the oracle collapse of that argmax, and the GPU
    decoder fed one-hot logits of the oracle's argmax reproduces the
    oracle's ids).
Rows of a batch are independent, so at the full workload sizes the GPU runs
the whole batch in the benchmark's launch configuration and the oracle
computes sampled rows.
"""
import functools
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def _inputs(cfg):
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    return W, pcm, valid


@functools.lru_cache(maxsize=None)
def _oracle(cfg, rows):
    W, pcm, valid = _inputs(cfg)
    rows = list(rows)
    lg, vf = oracle.forward(cfg.replace(batch=len(rows)), W, pcm[rows], valid[rows])
    return lg, vf


def _gpu_forward(cfg, precision=None, pcm=None, valid=None):
    import wav2vec2_ctc_encoder_amd as w2
    W, pcm0, valid0 = _inputs(cfg)
    pcm = pcm0 if pcm is None else pcm
    valid = valid0 if valid is None else valid
    with w2.Model(cfg, W, max_batch=pcm.shape[0], precision=precision) as m:
        tp = torch.from_numpy(pcm).cuda()
        tv = torch.from_numpy(valid).cuda()
        logits, vf = m.forward(tp, tv)
        ids, lens = w2.ctc_greedy(logits, vf, blank_id=cfg.blank_id)
        torch.cuda.synchronize()
        return logits.cpu().numpy(), vf.cpu().numpy(), ids.cpu().numpy(), lens.cpu().numpy()


def _pearson(a, b):
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    a -= a.mean()
    b -= b.mean()
    return float((a @ b) / np.sqrt((a @ a) * (b @ b)))


def _check_ids(cfg, logits, vf, ids, lens):
    """GPU ids equal the oracle's collapse of the GPU argmax."""
    a = oracle.frame_argmax(logits)
    for b in range(logits.shape[0]):
        want = oracle.ctc_collapse(a[b, :vf[b]], cfg.blank_id)
        assert lens[b] == len(want), (b, lens[b], len(want))
        assert np.array_equal(ids[b, :lens[b]], want), b
        assert np.all(ids[b, lens[b]:] == -1)


def _gate_fp32(gpu, ref):
    err = np.abs(gpu.astype(np.float64) - ref).max()
    _say(f"fp32 max-abs {err:.3e}")
    assert err <= 1e-3, err


def _row_mismatch_limit(n):
    # Per-row check beside the pooled gate: at most max(2, 1% of the row's
    # frames) mismatched frames.  A CPU emulation of this path's fp16 rounding
    # points on the large workload puts single 799-frame rows between 99.37%
    # and 100% (1 frame = 0.125%), the flips falling on frames whose top-2
    # logit margin is below the fp16-mode logit error.
    return max(2, int(np.ceil(0.01 * n)))


def _gate_fp16(gpu, ref, vf):
    """Pooled over the sampled rows (as the TensorRT README's quality table
    pools its clips): Pearson >= 0.999 and argmax agreement >= 99.5%; every
    row within _row_mismatch_limit."""
    per = []
    for i in range(len(vf)):
        n = int(vf[i])
        mis = int(np.sum(np.argmax(gpu[i, :n], -1) != np.argmax(ref[i, :n], -1)))
        per.append((n, mis))
    sel_g = np.concatenate([gpu[i, :vf[i]] for i in range(len(vf))])
    sel_r = np.concatenate([ref[i, :vf[i]] for i in range(len(vf))])
    r = _pearson(sel_g, sel_r)
    agree = float(np.mean(np.argmax(sel_g, -1) == np.argmax(sel_r, -1)))
    rows = ", ".join(f"{1 - m / n if n else 1:.5f} ({m}/{n})" for n, m in per)
    _say(f"fp16 pearson {r:.6f} argmax agreement {agree:.5f} over {len(sel_g)} frames; per row {rows}")
    assert r >= 0.999, r
    assert agree >= 0.995, agree
    for n, m in per:
        assert m <= _row_mismatch_limit(n), (n, m)
    return agree


def _ids_given_oracle_argmax(cfg, ref, vf):
    """Feed one-hot logits of the oracle's argmax to the GPU decoder."""
    import wav2vec2_ctc_encoder_amd as w2
    a = oracle.frame_argmax(ref)
    B, T = a.shape
    onehot = np.full((B, T, cfg.vocab), -1.0, np.float32)
    np.put_along_axis(onehot, a[..., None].astype(np.int64), 1.0, axis=-1)
    ids, lens = w2.ctc_greedy(torch.from_numpy(onehot).cuda(), torch.from_numpy(vf.astype(np.int32)).cuda(),
                              blank_id=cfg.blank_id)
    ids, lens = ids.cpu().numpy(), lens.cpu().numpy()
    want = oracle.greedy_decode(ref, vf, cfg.blank_id)
    for b in range(B):
        assert np.array_equal(ids[b, :lens[b]], want[b]), b


# ----------------------------------------------------------------------------
# tiny network, whole oracle
# ----------------------------------------------------------------------------
_TINY = synth.TINY_1S_B1
_TINY_VARIANTS = {
    "group_postnorm": _TINY,
    "layer_stable_bias": _TINY.replace(feat_norm="layer", conv_bias=True, stable_layer_norm=True),
    "group_bias_odd_pos_kernel": _TINY.replace(conv_bias=True, pos_kernel=15),
    "ragged_batch3": _TINY.replace(batch=3, valid_range=(300, 16000), pcm_seed=777),
    "head32_window_tail": _TINY.replace(hidden=128, heads=4, window=16000 + 3333, batch=2,
                                        valid_range=(9000, 19333)),
    "head128": _TINY.replace(hidden=256, heads=2, ffn=512, pos_groups=8),
    # d_h = 64 (the base and large head size) over 153 frames: two query
    # blocks of 128 and three key tiles of 64, both with a ragged tail
    "head64_ragged_tiles": _TINY.replace(hidden=128, heads=2, window=3 * 16000 + 1234, batch=3,
                                         valid_range=(300, 3 * 16000 + 1234)),
    # d_h = 64 over 40 s windows: 1999 frames, 16 query blocks and 32 key
    # tiles per (row, head), longer than any benchmark workload
    "head64_long_window": _TINY.replace(hidden=128, heads=2, window=40 * 16000, batch=2,
                                        valid_range=(20 * 16000, 40 * 16000)),
    "tanh_gelu_group": _TINY.replace(gelu="tanh", batch=2, valid_range=(8000, 16000)),
    "tanh_gelu_layer_stable": _TINY.replace(gelu="tanh", feat_norm="layer", conv_bias=True, stable_layer_norm=True),
}


@pytest.mark.parametrize("variant", sorted(_TINY_VARIANTS))
def test_tiny_fp32_matches_oracle(variant):
    cfg = _TINY_VARIANTS[variant]
    _say(f"tiny fp32 {variant}")
    ref, vf_ref = _oracle(cfg, tuple(range(cfg.batch)))
    logits, vf, ids, lens = _gpu_forward(cfg, precision="fp32")
    assert np.array_equal(vf, vf_ref)
    _gate_fp32(logits, ref)
    _check_ids(cfg, logits, vf, ids, lens)
    _ids_given_oracle_argmax(cfg, ref, vf_ref)


@pytest.mark.parametrize("variant", ["group_postnorm", "layer_stable_bias", "head64_ragged_tiles",
                                     "head64_long_window"])
def test_tiny_fp16_correlates(variant):
    cfg = _TINY_VARIANTS[variant]
    _say(f"tiny fp16 {variant}")
    ref, vf_ref = _oracle(cfg, tuple(range(cfg.batch)))
    logits, vf, ids, lens = _gpu_forward(cfg, precision="fp16")
    r = _pearson(logits, ref)
    _say(f"pearson {r:.6f}")
    assert r >= 0.999
    _check_ids(cfg, logits, vf, ids, lens)


def test_tanh_gelu_mode_on_base_shape():
    """The tanh-GELU compatibility mode at the base 10 s shape in fp16 meets
    the fp16 gates against the tanh-GELU oracle, and its deviation from the
    exact-GELU network is reported."""
    cfg = synth.BASE_10S_B1.replace(gelu="tanh", window=96000)
    _say("base 6 s tanh-GELU fp16")
    ref, vf_ref = _oracle(cfg, (0,))
    logits, vf, ids, lens = _gpu_forward(cfg, precision="fp16")
    _gate_fp16(logits, ref, vf_ref)
    ref_erf, _ = _oracle(cfg.replace(gelu="erf"), (0,))
    _say(f"tanh-vs-erf network: max-abs {np.abs(ref - ref_erf).max():.3e}, "
         f"pearson {_pearson(ref, ref_erf):.6f}, "
         f"argmax agreement {np.mean(np.argmax(ref[0, :vf_ref[0]], -1) == np.argmax(ref_erf[0, :vf_ref[0]], -1)):.4f}")


@pytest.mark.parametrize("dc", [0.5, -2.0])
def test_dc_offset_pcm(dc):
    """GroupNorm statistics under a large DC offset (the variance is small
    next to the mean): fp32 gate against the oracle."""
    import wav2vec2_ctc_encoder_amd as w2
    cfg = _TINY.replace(batch=2, valid_range=(12000, 16000))
    _say(f"pcm + DC {dc}")
    W, pcm, valid = _inputs(cfg)
    pcm = pcm.copy()
    for b in range(cfg.batch):
        pcm[b, :valid[b]] += np.float32(dc)
    ref, vf_ref = oracle.forward(cfg, W, pcm, valid)
    logits, vf, ids, lens = _gpu_forward(cfg, precision="fp32", pcm=pcm, valid=valid)
    _gate_fp32(logits, ref)


def test_samples_beyond_valid_are_ignored():
    import wav2vec2_ctc_encoder_amd as w2
    cfg = _TINY_VARIANTS["ragged_batch3"]
    _say("garbage beyond valid length")
    W, pcm, valid = _inputs(cfg)
    pcm_g, _ = synth.make_pcm(cfg, valid=valid, pad_garbage=True)
    a = _gpu_forward(cfg, precision="fp32")[0]
    b = _gpu_forward(cfg, precision="fp32", pcm=pcm_g, valid=valid)[0]
    assert np.array_equal(a, b)


def test_short_and_empty_rows():
    cfg = _TINY.replace(batch=4, rand_affine=False)
    _say("valid lengths 0, 399, 400, window")
    valid = np.array([0, 399, 400, cfg.window], np.int32)
    W = synth.make_weights(cfg)
    pcm, _ = synth.make_pcm(cfg, valid=valid)
    ref, vf_ref = oracle.forward(cfg, W, pcm, valid)
    import wav2vec2_ctc_encoder_amd as w2
    with w2.Model(cfg, W, precision="fp32") as m:
        logits, vf = m.forward(torch.from_numpy(pcm).cuda(), torch.from_numpy(valid).cuda())
        ids, lens = w2.ctc_greedy(logits, vf, blank_id=0)
        logits, vf, ids, lens = (x.cpu().numpy() for x in (logits, vf, ids, lens))
    assert vf.tolist() == [0, 0, 1, 49] == vf_ref.tolist()
    assert lens[0] == 0 and lens[1] == 0 and np.all(ids[:2] == -1)
    _gate_fp32(logits, ref)
    _check_ids(cfg, logits, vf, ids, lens)


def test_all_zero_pcm_gives_zero_logits_on_gpu():
    """Zero PCM, zero biases, unit gains: the network maps 0 to exactly 0."""
    import wav2vec2_ctc_encoder_amd as w2
    for prec in ("fp32", "fp16"):
        for cfg in (_TINY.replace(rand_affine=False, batch=2),
                    _TINY.replace(rand_affine=False, batch=2, feat_norm="layer", stable_layer_norm=True)):
            _say(f"zero pcm {prec} {cfg.feat_norm}")
            W = synth.make_weights(cfg)
            with w2.Model(cfg, W, precision=prec) as m:
                pcm = torch.zeros(2, cfg.window, device="cuda")
                valid = torch.tensor([cfg.window, 5000], dtype=torch.int32, device="cuda")
                logits, vf = m.forward(pcm, valid)
                ids, lens = w2.ctc_greedy(logits, vf)
                assert torch.count_nonzero(logits).item() == 0
                assert lens.cpu().tolist() == [0, 0]


def test_frontend_and_encoder_stages_tiny():
    import wav2vec2_ctc_encoder_amd as w2
    cfg = _TINY_VARIANTS["ragged_batch3"]
    _say("stage split tiny fp32")
    W, pcm, valid = _inputs(cfg)
    feats_ref = oracle.feature_encoder(cfg, W, pcm, valid).transpose(0, 2, 1)       # [B, T, C]
    logits_ref = oracle.ctc_head(W, oracle.encoder(cfg, W, feats_ref.transpose(0, 2, 1)))
    with w2.Model(cfg, W, precision="fp32") as m:
        f = m.forward_frontend(torch.from_numpy(pcm).cuda(), torch.from_numpy(valid).cuda())
        err_f = np.abs(f.cpu().numpy() - feats_ref).max()
        lg = m.forward_encoder(torch.from_numpy(np.ascontiguousarray(feats_ref, dtype=np.float32)).cuda())
        err_e = np.abs(lg.cpu().numpy() - logits_ref).max()
    _say(f"frontend max-abs {err_f:.3e} encoder max-abs {err_e:.3e}")
    assert err_f <= 1e-4
    assert err_e <= 1e-3


# ----------------------------------------------------------------------------
# CTC decoder on hand-built logits
# ----------------------------------------------------------------------------
def test_ctc_greedy_fake_engine_paths():
    import wav2vec2_ctc_encoder_amd as w2
    _say("ctc fake engine")
    rng = np.random.default_rng(3)
    B, T, V = 6, 1500, 37
    paths = rng.integers(0, V, size=(B, T)).astype(np.int32)
    paths[1, :] = 0
    paths[2, ::2] = 5
    paths[2, 1::2] = 5
    vf = np.array([T, T, 999, 1, 0, 1024], np.int32)
    logits = rng.standard_normal((B, T, V)).astype(np.float32)
    np.put_along_axis(logits, paths[..., None].astype(np.int64), 10.0, axis=-1)
    ids, lens = w2.ctc_greedy(torch.from_numpy(logits).cuda(), torch.from_numpy(vf).cuda(), blank_id=0)
    ids, lens = ids.cpu().numpy(), lens.cpu().numpy()
    for b in range(B):
        want = oracle.ctc_collapse(paths[b, :vf[b]], 0)
        assert lens[b] == len(want)
        assert np.array_equal(ids[b, :lens[b]], want)
        assert np.all(ids[b, lens[b]:] == -1)


def test_ctc_argmax_ties_and_large_vocab():
    import wav2vec2_ctc_encoder_amd as w2
    _say("argmax ties, vocab 2341, blank 7")
    rng = np.random.default_rng(4)
    B, T, V = 3, 50, 2341
    logits = np.round(rng.standard_normal((B, T, V)) * 2).astype(np.float32)  # many exact ties
    vf = np.array([50, 17, 49], np.int32)
    ids, lens = w2.ctc_greedy(torch.from_numpy(logits).cuda(), torch.from_numpy(vf).cuda(), blank_id=7)
    ids, lens = ids.cpu().numpy(), lens.cpu().numpy()
    want = oracle.greedy_decode(logits, vf, 7)
    for b in range(B):
        assert np.array_equal(ids[b, :lens[b]], want[b])


# ----------------------------------------------------------------------------
# full workloads (oracle on sampled rows)
# ----------------------------------------------------------------------------
_FULL = {
    "base_10s_b1": (synth.BASE_10S_B1, (0,)),
    # rows 2 and 4 hold 5.6 s and 3.4 s of audio in the 16 s window
    "base_16s_b8": (synth.BASE_16S_B8, (0, 2, 4, 5)),
    "large_16s_b4": (synth.LARGE_16S_B4, (0, 1, 2, 3)),
    "base_16s_b32": (synth.BASE_16S_B32, (0, 31)),
}


@pytest.mark.parametrize("name", list(_FULL))
def test_full_workload_fp16(name):
    cfg, rows = _FULL[name]
    _say(f"{name} fp16 rows {rows}")
    ref, vf_ref = _oracle(cfg, rows)
    logits, vf, ids, lens = _gpu_forward(cfg, precision="fp16")
    r = list(rows)
    assert np.array_equal(vf[r], vf_ref)
    _gate_fp16(logits[r], ref, vf_ref)
    _check_ids(cfg, logits, vf, ids, lens)
    _ids_given_oracle_argmax(cfg, ref, vf_ref)
    assert np.isfinite(logits).all()


@pytest.mark.parametrize("name", ["base_10s_b1", "base_16s_b8", "large_16s_b4"])
def test_full_workload_fp32(name):
    cfg, rows = _FULL[name]
    _say(f"{name} fp32 rows {rows}")
    ref, vf_ref = _oracle(cfg, rows)
    logits, vf, ids, lens = _gpu_forward(cfg, precision="fp32")
    _gate_fp32(logits[list(rows)], ref)
    _check_ids(cfg, logits, vf, ids, lens)


@pytest.mark.parametrize("conv_bias", [False, True])
def test_base_rand_affine_fp16(conv_bias):
    """Every norm gain/shift, bias and weight-norm gain random at base size
    (512 feature channels: the matrix-core conv0 of the group-norm layout,
    with and without a conv bias folded into the GroupNorm shift)."""
    cfg = synth.BASE_10S_B1.replace(rand_affine=True, window=64000, weight_seed=99, conv_bias=conv_bias)
    _say(f"base 4 s rand_affine fp16 conv_bias={conv_bias}")
    ref, vf_ref = _oracle(cfg, (0,))
    logits, vf, ids, lens = _gpu_forward(cfg, precision="fp16")
    _gate_fp16(logits, ref, vf_ref)


def test_deterministic_and_batch_permutation():
    import wav2vec2_ctc_encoder_amd as w2
    cfg = synth.BASE_16S_B8
    _say("determinism + permutation base_16s_b8 fp16")
    W, pcm, valid = _inputs(cfg)
    perm = [3, 0, 7, 1, 6, 2, 5, 4]
    with w2.Model(cfg, W) as m:
        tp, tv = torch.from_numpy(pcm).cuda(), torch.from_numpy(valid).cuda()
        a, _ = m.forward(tp, tv)
        a = a.clone()
        b, _ = m.forward(tp, tv)
        assert torch.equal(a, b)
        c, _ = m.forward(tp[perm].contiguous(), tv[perm].contiguous())
        assert torch.equal(c, a[perm])
        # a smaller batch in the same model gives the same rows
        d, _ = m.forward(tp[:3].contiguous(), tv[:3].contiguous())
        assert torch.equal(d, a[:3])


@pytest.mark.parametrize("batch", [2, 5])
def test_two_stream_split_matches_one_pass(batch):
    # batch >= 2 runs its halves concurrently on two streams; profiling every
    # kernel runs it as one pass on one stream: the bits must agree
    import wav2vec2_ctc_encoder_amd as w2
    cfg = synth.BASE_10S_B1.replace(batch=batch, layers=2, valid_range=(20000, 160000), pcm_seed=4242)
    _say(f"two-stream split vs one pass, batch {batch}")
    W, pcm, valid = _inputs(cfg)
    with w2.Model(cfg, W, max_batch=batch) as m:
        tp, tv = torch.from_numpy(pcm).cuda(), torch.from_numpy(valid).cuda()
        split, vf_split = m.forward(tp, tv)
        m.profile_enable(True)
        one, vf_one = m.forward(tp, tv)
        torch.cuda.synchronize()
        m.profile_read()
        m.profile_enable(False)
        assert torch.equal(vf_split, vf_one)
        assert torch.equal(split, one)


# ----------------------------------------------------------------------------
# forward + decode in one call (argmax inside the CTC head's epilogue)
# ----------------------------------------------------------------------------
def _fused_vs_separate(cfg, W, pcm, valid, precision=None):
    import wav2vec2_ctc_encoder_amd as w2
    with w2.Model(cfg, W, max_batch=pcm.shape[0], precision=precision) as m:
        tp, tv = torch.from_numpy(pcm).cuda(), torch.from_numpy(valid).cuda()
        lg, vf = m.forward(tp, tv)
        ids, lens = w2.ctc_greedy(lg, vf, blank_id=cfg.blank_id)
        lg2, vf2, ids2, lens2 = m.forward_greedy(tp, tv)
        torch.cuda.synchronize()
        assert torch.equal(lg, lg2)
        assert torch.equal(vf, vf2)
        assert torch.equal(lens, lens2)
        assert torch.equal(ids, ids2)
        return lg2.cpu().numpy(), vf2.cpu().numpy(), ids2.cpu().numpy(), lens2.cpu().numpy()


# the head's three epilogue paths: 16x16 register-staged kernel (N <= 32 or
# fp32), the 32x32 kernel's LDS-staged epilogue (N % 8 == 0) and its direct
# epilogue (N = 2341)
_FUSED_TINY = {
    "v32_fp32": (_TINY, "fp32"),
    "v32_fp16": (_TINY, "fp16"),
    "v256_fp16_staged": (_TINY.replace(vocab=256, batch=3, valid_range=(400, 16000)), "fp16"),
    "v2341_fp16_direct": (_TINY.replace(vocab=2341, batch=2, valid_range=(6000, 16000)), "fp16"),
    "v2341_fp32": (_TINY.replace(vocab=2341, batch=2, valid_range=(6000, 16000)), "fp32"),
}


@pytest.mark.parametrize("variant", sorted(_FUSED_TINY))
def test_forward_greedy_tiny_matches_separate_decode(variant):
    cfg, prec = _FUSED_TINY[variant]
    _say(f"forward_greedy tiny {variant}")
    W, pcm, valid = _inputs(cfg)
    lg, vf, ids, lens = _fused_vs_separate(cfg, W, pcm, valid, prec)
    _check_ids(cfg, lg, vf, ids, lens)


@pytest.mark.parametrize("name", ["base_10s_b1", "base_16s_b8", "large_16s_b4", "base_16s_b32"])
def test_forward_greedy_full_workloads_match_separate_decode(name):
    cfg = synth.PRESETS[name]
    _say(f"forward_greedy {name}")
    W, pcm, valid = _inputs(cfg)
    _fused_vs_separate(cfg, W, pcm, valid)


@pytest.mark.parametrize("prec", ["fp32", "fp16"])
@pytest.mark.parametrize("vocab", [32, 2341])
def test_forward_greedy_exact_ties_and_signed_zeros(prec, vocab):
    """Zero head weight: every frame's logits equal the head bias exactly.
    The bias holds its maximum three times and -0 / +0 side by side, so the
    argmax must be the first maximum; with the maximum at 0 (-0 first) the
    -0 and +0 entries tie."""
    cfg = _TINY.replace(vocab=vocab, batch=2, valid_range=(9000, 16000))
    W, pcm, valid = _inputs(cfg)
    for top, first in ((3.0, 5), (0.0, 2)):
        _say(f"forward_greedy ties {prec} V={vocab} max={top}")
        W2 = dict(W)
        W2["head.weight"] = np.zeros_like(W["head.weight"])
        bias = np.full(vocab, -1.0, np.float32)
        if top > 0:
            bias[[5, 9, vocab - 1]] = top
            bias[2] = -0.0
            bias[7] = 0.0
        else:
            bias[2] = -0.0
            bias[7] = 0.0
            bias[vocab - 3] = 0.0
        W2["head.bias"] = bias
        lg, vf, ids, lens = _fused_vs_separate(cfg, W2, pcm, valid, prec)
        a = oracle.frame_argmax(lg)
        assert np.all(a[:, :] == first), np.unique(a)
        for b in range(cfg.batch):
            assert lens[b] == (1 if vf[b] > 0 else 0)
            if vf[b] > 0:
                assert ids[b, 0] == first


@pytest.mark.parametrize("name,batch", [("base_10s_b1", 1), ("base_10s_b1", 3)])
def test_forward_greedy_graph_replays_match_eager(name, batch):
    """forward_greedy captured once into a HIP graph (one stream for batch 1,
    the forked second stream for batch 3) and replayed several times, with
    eager calls on other inputs and synchronizations between the replays:
    every replay gives the eager call's exact logits and ids."""
    import wav2vec2_ctc_encoder_amd as w2
    cfg = synth.PRESETS[name].replace(batch=batch, layers=2, valid_range=(20000, 160000), pcm_seed=909)
    _say(f"graph replay forward_greedy {name} batch {batch}")
    W, pcm, valid = _inputs(cfg)
    other = np.flip(pcm, axis=1).copy()  # other samples, same valid lengths
    with w2.Model(cfg, W, max_batch=batch) as m:
        tp, tv = torch.from_numpy(pcm).cuda(), torch.from_numpy(valid).cuda()
        to = torch.from_numpy(other).cuda()
        ref = [t.clone() for t in m.forward_greedy(tp, tv)]
        bufs = [torch.empty_like(t) for t in ref]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            m.forward_greedy(tp, tv, *bufs)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            m.forward_greedy(tp, tv, *bufs)
        torch.cuda.synchronize()
        for it in range(4):
            for b in bufs:
                b.fill_(-7)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for r, b in zip(ref, bufs):
                assert torch.equal(r, b), it
            # eager work on other inputs between the replays
            m.forward_greedy(to, tv)
            torch.cuda.synchronize()


def test_workspace_beyond_device_memory_is_nomem():
    """A max_batch whose workspace exceeds the device's memory fails at
    create with W2V2_E_NOMEM (4096 windows of 16 s need about 390 GB), and
    the library stays usable."""
    import wav2vec2_ctc_encoder_amd as w2
    cfg = synth.BASE_16S_B8.replace(layers=1)
    W = synth.make_weights(cfg)
    _say("max_batch 4096 x 16 s: out of device memory")
    with pytest.raises(w2.W2V2Error) as e:
        w2.Model(cfg, W, max_batch=4096)
    assert e.value.status == 4  # W2V2_E_NOMEM
    with w2.Model(cfg.replace(batch=1), W, max_batch=1) as m:
        pcm, valid = synth.make_pcm(cfg.replace(batch=1))
        lg, vf = m.forward(torch.from_numpy(pcm).cuda(), torch.from_numpy(valid).cuda())
        torch.cuda.synchronize()
        assert vf.item() == int(oracle.valid_frames(cfg, valid)[0]) and torch.isfinite(lg).all()
