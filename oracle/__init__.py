"""CPU oracle of wav2vec2-CTC encoder inference (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  See ``w2v2_oracle`` for the definitions and sources.
"""
from .w2v2_oracle import (  # noqa: F401
    E4M3_MAX, FP8_INPUTS, activation, amax_key, calibrate_amax, conv1d, conv_out_len, ctc_collapse, ctc_head, encoder, feature_encoder, feed_forward,
    fold_weight_norm, forward, forward_true_length, frame_argmax, gelu, gelu_tanh, greedy_decode, group_norm_over_time,
    layer_norm, linear, num_frames, positional_conv, quantize_e4m3, self_attention, softmax, valid_frames,
)
