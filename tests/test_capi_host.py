"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and validates arguments before touching a device."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w2v2.h")


def _lib():
    from wav2vec2_ctc_encoder_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libw2v2.so is not built (run __graft_entry__.build())")
    return L


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w2v2_[a-z_]+)\s*\(", text)))


def test_header_declares_the_documented_entry_points():
    syms = _declared_symbols()
    for s in ("w2v2_create", "w2v2_forward", "w2v2_ctc_greedy", "w2v2_destroy", "w2v2_last_error"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    L = _lib()
    so = ctypes.CDLL(L.LIB_PATH)
    missing = [s for s in _declared_symbols() if not hasattr(so, s)]
    assert not missing, missing
    assert set(L.EXPORTED) == set(_declared_symbols())


def test_binding_names_match_header_struct_fields():
    """ctypes structs mirror the header structs field by field."""
    L = _lib()
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} w2v2_config;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"\b([a-z_]+)(?:\[[A-Z_0-9]+\])?;", body)
    assert [f for f, _ in L.Config._fields_] == fields


def _config(**kw):
    from wav2vec2_ctc_encoder_amd import make_config
    cfg = synth.TINY_1S_B1.replace(**kw)
    return cfg, make_config(cfg)


def _create(cfg_struct, weights):
    L = _lib()
    lib = L.lib()
    arrays = {k: np.ascontiguousarray(v, np.float32) for k, v in weights.items()}
    names = [k.encode() for k in arrays]
    tab = (L.Tensor * max(1, len(arrays)))()
    for i, (k, a) in enumerate(arrays.items()):
        tab[i].name = names[i]
        tab[i].data = a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
        tab[i].ndim = a.ndim
        for j, s in enumerate(a.shape):
            tab[i].shape[j] = s
    h = ctypes.c_void_p(123)
    st = lib.w2v2_create(ctypes.byref(cfg_struct), tab, len(arrays), 0, ctypes.byref(h))
    return st, h, lib.w2v2_last_error().decode()


@pytest.mark.parametrize("field,value", [
    ("abi_version", 99), ("n_conv", 0), ("n_conv", 9), ("heads", 5), ("heads", 64), ("ffn", 12),
    ("pos_groups", 3), ("vocab", 0), ("blank_id", 32), ("blank_id", -1), ("eps", 0.0),
    ("precision", 7), ("max_batch", 0), ("max_batch", 5000), ("window", 399), ("feat_norm", 3),
    ("gelu_kind", 2), ("sample_rate", 8000), ("precision", 2), ("precision", 3),
])
def test_bad_config_rejected_before_device_work(field, value):
    cfg, c = _config()
    setattr(c, field, value)
    st, h, msg = _create(c, synth.make_weights(cfg))
    L = _lib()
    assert st == L.E_CONFIG, (st, msg)
    assert h.value is None
    assert msg


def test_bad_conv_dims_rejected():
    cfg, c = _config()
    c.conv_dim[2] = 36  # not a multiple of 8
    st, _, msg = _create(c, synth.make_weights(cfg))
    assert st == _lib().E_CONFIG, msg


@pytest.mark.parametrize("field,index,value", [("conv_dim", 0, 520), ("conv_kernel", 0, 17),
                                               ("conv_stride", 0, 9), ("conv_kernel", 3, 0)])
def test_unsupported_conv0_limits_rejected(field, index, value):
    cfg, c = _config()
    getattr(c, field)[index] = value
    st, _, msg = _create(c, synth.make_weights(cfg))
    assert st == _lib().E_CONFIG, msg


@pytest.mark.parametrize("case", ["empty", "missing", "extra", "duplicate", "shape", "nonfinite"])
def test_bad_weight_table_rejected(case):
    cfg, c = _config()
    W = synth.make_weights(cfg)
    if case == "empty":
        W = {}
    elif case == "missing":
        W.pop("layer1.ffn.fc2.bias")
    elif case == "extra":
        W["layer9.attn.q.weight"] = np.zeros((64, 64), np.float32)
    elif case == "shape":
        W["head.weight"] = np.zeros((33, 64), np.float32)
    elif case == "nonfinite":
        W["pos.bias"] = W["pos.bias"].copy()
        W["pos.bias"][3] = np.nan
    if case == "duplicate":
        L = _lib()
        lib = L.lib()
        items = list(W.items()) + [("head.bias", W["head.bias"])]
        tab = (L.Tensor * len(items))()
        keep = []
        for i, (k, a) in enumerate(items):
            a = np.ascontiguousarray(a, np.float32)
            keep.append((k.encode(), a))
            tab[i].name = keep[-1][0]
            tab[i].data = a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
            tab[i].ndim = a.ndim
            for j, s in enumerate(a.shape):
                tab[i].shape[j] = s
        h = ctypes.c_void_p()
        st = lib.w2v2_create(ctypes.byref(c), tab, len(items), 0, ctypes.byref(h))
        assert st == L.E_WEIGHTS
        assert "duplicate" in lib.w2v2_last_error().decode()
        return
    st, h, msg = _create(c, W)
    assert st == _lib().E_WEIGHTS, (st, msg)


def test_weight_norm_gain_shape_1_1_K_accepted_by_validation():
    """pos.weight_g may be [K] or [1, 1, K]; validation passes either way
    (with no GPU the call then fails at the device step, not on weights)."""
    cfg, c = _config()
    W = synth.make_weights(cfg)
    W["pos.weight_g"] = W["pos.weight_g"].reshape(1, 1, -1)
    st, _, msg = _create(c, W)
    L = _lib()
    assert st in (L.OK, L.E_DEVICE), msg


def test_null_arguments_rejected():
    L = _lib()
    lib = L.lib()
    h = ctypes.c_void_p()
    assert lib.w2v2_create(None, None, 0, 0, ctypes.byref(h)) == L.E_ARG
    assert lib.w2v2_forward(None, None, None, 1, None, None, None) == L.E_ARG
    assert lib.w2v2_forward_true_length(None, None, None, 1, None, None, None) == L.E_ARG
    assert lib.w2v2_forward_frontend(None, None, None, 1, None, None) == L.E_ARG
    assert lib.w2v2_forward_encoder(None, None, 1, None, None) == L.E_ARG
    assert lib.w2v2_forward_greedy(None, None, None, 1, None, None, None, None, None) == L.E_ARG
    assert lib.w2v2_calibrate(None, None, None, 1, None, None, None) == L.E_ARG
    assert lib.w2v2_ctc_greedy(None, None, 1, 10, 32, 0, None, None, None) == L.E_ARG
    # valid-looking pointers but bad sizes (no device access happens)
    p = ctypes.c_void_p(0x1000)
    assert lib.w2v2_ctc_greedy(p, p, 0, 10, 32, 0, p, p, None) == L.E_ARG
    assert lib.w2v2_ctc_greedy(p, p, 1, 0, 32, 0, p, p, None) == L.E_ARG
    assert lib.w2v2_ctc_greedy(p, p, 1, 20000, 32, 0, p, p, None) == L.E_ARG
    assert lib.w2v2_ctc_greedy(p, p, 1, 10, 32, 32, p, p, None) == L.E_ARG
    n = ctypes.c_int32()
    assert lib.w2v2_num_frames(None, 16000, ctypes.byref(n)) == L.E_ARG
    assert lib.w2v2_profile_enable(None, 1, None) == L.E_ARG
    assert lib.w2v2_last_error().decode() != ""


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from wav2vec2_ctc_encoder_amd import _lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(L.LibraryMissing):
        L.lib()


def _fp8_case(**kw):
    """A tiny network the fp8 modes accept (hidden and ffn multiples of 128)."""
    from wav2vec2_ctc_encoder_amd import make_config
    cfg = synth.TINY_1S_B1.replace(hidden=128, heads=4, ffn=256, **kw)
    W = synth.make_weights(cfg)
    for l in range(cfg.layers):
        for w in ("attn.qkv", "attn.out", "ffn.fc1", "ffn.fc2"):
            W[f"layer{l}.{w}.input_amax"] = np.array([2.5], np.float32)
    return cfg, W, make_config(cfg)


@pytest.mark.parametrize("prec", [2, 3])
def test_fp8_weight_table_validation(prec):
    L = _lib()
    cfg, W, c = _fp8_case()
    c.precision = prec
    # a complete table passes validation: with no GPU the call stops at the device
    st, _, msg = _create(c, W)
    assert st in (L.OK, L.E_DEVICE), msg
    for case in ("missing", "zero", "negative", "shape"):
        W2 = dict(W)
        key = "layer1.ffn.fc2.input_amax"
        if case == "missing":
            W2.pop(key)
        elif case == "zero":
            W2[key] = np.array([0.0], np.float32)
        elif case == "negative":
            W2[key] = np.array([-1.0], np.float32)
        else:
            W2[key] = np.array([1.0, 2.0], np.float32)
        st, _, msg = _create(c, W2)
        assert st == L.E_WEIGHTS, (case, st, msg)
    # the fp16 / fp32 modes take no amax entries
    c.precision = 1
    st, _, msg = _create(c, W)
    assert st == L.E_WEIGHTS and "unknown weight" in msg


def test_no_device_is_a_device_error():
    """With a valid config and weight table and no HIP device, create fails
    with W2V2_E_DEVICE (this container has no GPU)."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    cfg, c = _config()
    st, h, msg = _create(c, synth.make_weights(cfg))
    assert st == _lib().E_DEVICE, (st, msg)
    assert h.value is None and "device" in msg.lower()


def test_amax_table_names_match_the_oracle():
    import oracle
    from wav2vec2_ctc_encoder_amd import FP8_INPUTS, amax_table
    assert tuple(FP8_INPUTS) == tuple(oracle.FP8_INPUTS)
    t = amax_table(np.arange(8, dtype=np.float32).reshape(2, 4) + 1)
    assert t["layer1.ffn.fc1.input_amax"][0] == 7.0
    assert sorted(t) == sorted(oracle.amax_key(l, w) for l in range(2) for w in oracle.FP8_INPUTS)
