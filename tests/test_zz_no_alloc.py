"""w2v2_forward_greedy_noalloc (every intermediate in the library's static
device scratch) against w2v2_forward_greedy (the model's workspace): bitwise
identical logits, frames, ids and lengths on two calls in a row, the second
with a smaller batch, and rejection of a batch that does not fit the scratch.
"""
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _outputs(m, B):
    T = m.frames_per_window
    return (torch.empty(B, T, m.vocab, dtype=torch.float32, device="cuda"),
            torch.empty(B, dtype=torch.int32, device="cuda"),
            torch.empty(B, T, dtype=torch.int32, device="cuda"),
            torch.empty(B, dtype=torch.int32, device="cuda"))


@pytest.mark.parametrize("name", ["tiny", "base_1s", "base_1s_fp8"])
def test_noalloc_matches_forward_greedy(name):
    import wav2vec2_ctc_encoder_amd as w2
    if name == "tiny":
        cfg, prec = synth.TINY_1S_B1.replace(batch=5, valid_range=(300, 16000)), "fp32"
    else:
        cfg, prec = synth.BASE_10S_B1.replace(window=16000, batch=6, valid_range=(300, 16000), pcm_seed=77), "fp16"
    W = synth.make_weights(cfg)
    if name == "base_1s_fp8":
        prec = "fp8"
        W = dict(W, **w2.amax_table(np.full((cfg.layers, 4), 3.0, np.float32)))
    pcm, valid = synth.make_pcm(cfg)
    _say(f"noalloc vs forward_greedy {name} {prec}")
    with w2.Model(cfg, W, max_batch=cfg.batch, precision=prec) as m:
        for B in (cfg.batch, 3):            # two calls in a row, the second smaller
            tp = torch.from_numpy(pcm[:B].copy()).cuda()
            tv = torch.from_numpy(valid[:B].copy()).cuda()
            ref = m.forward_greedy(tp, tv)
            out = _outputs(m, B)
            for t in out:
                t.fill_(-3)
            m.forward_greedy_noalloc(tp, tv, *out)
            torch.cuda.synchronize()
            for r, o in zip(ref, out):
                assert torch.equal(r, o), B


def test_noalloc_rejects_batches_beyond_the_scratch():
    import wav2vec2_ctc_encoder_amd as w2
    # a 16 s window's intermediates (conv0 output alone 52 MB) exceed the scratch
    cfg = synth.BASE_10S_B1.replace(layers=1, batch=1, window=256000)
    W = synth.make_weights(cfg)
    pcm, valid = synth.make_pcm(cfg)
    _say("noalloc rejects a 16 s window")
    with w2.Model(cfg, W, max_batch=1) as m:
        tp, tv = torch.from_numpy(pcm).cuda(), torch.from_numpy(valid).cuda()
        with pytest.raises(w2.W2V2Error, match="scratch"):
            m.forward_greedy_noalloc(tp, tv, *_outputs(m, 1))
        # the model still works afterwards
        lg, vf, ids, lens = m.forward_greedy(tp, tv)
        torch.cuda.synchronize()
        assert vf.item() == 799
