/*
 * w2v2.h - C ABI of the wav2vec2-CTC encoder inference library (gfx950).
 *
 * The library runs raw 16 kHz PCM windows through the 7-layer strided conv
 * feature encoder, the feature projection, the weight-norm grouped positional
 * conv, N transformer blocks and the CTC logit head on one AMD Instinct
 * MI355X (gfx950), and decodes the logits greedily into CTC token ids.
 * Every step runs in the library's own HIP kernels; there is no CPU fallback
 * and no other GPU target (an unsupported configuration or device fails at
 * w2v2_create).
 *
 * Sources, cited by page title and section:
 *  [LiteRT]  "litert-community/wav2vec2-base-960h-LiteRT - discussion #1":
 *            "Recipe" (config fields read from the checkpoint), "Rewrites for
 *            the GPU" (fixed zero-padded window, no attention mask, decoding
 *            over the valid frames, folded weight norm g*v/||v||, exact GELU).
 *  [TRT]     "TensorRT-Model-Connect families/wav2vec2 README":
 *            "Wav2Vec2 CTC layouts" (group-norm / per-frame layer-norm feature
 *            encoders with or without conv bias, post-norm or stable pre-norm
 *            blocks with the encoder norm after the blocks, validated
 *            non-empty weight table), "FP8 quantization study" (fp16 graph:
 *            convolutions, projections and attention in fp16, every
 *            normalization in fp32), "Recipe that was measured" (the
 *            projections and convolutions of the network), "Method" and
 *            "Results" (per-frame argmax, CTC token ids).
 *
 * Conventions common to all calls
 *  - Status codes are returned, never exceptions; w2v2_last_error() gives a
 *    human-readable message for the last failing call on this thread.
 *  - Every checkable argument is validated before any device work.
 *  - "dev" pointers are HIP device pointers on the model's device, owned by
 *    the caller; "host" pointers are ordinary host memory, owned by the
 *    caller.  The library never frees caller memory.
 *  - `stream` is a hipStream_t (NULL = the null stream) of the model's
 *    device.  Calls only enqueue work on it: they neither synchronize nor
 *    allocate, so results are ready when the caller synchronizes the stream.
 *    Asynchronous device faults surface at that synchronization.
 *  - A model's workspace is shared by its calls: calls on one model must be
 *    serialized (one stream at a time, or ordered by the caller).
 *  - Results are deterministic: the same inputs on the same model give
 *    bitwise identical outputs.
 */
#ifndef W2V2_H
#define W2V2_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W2V2_ABI_VERSION 2
#define W2V2_MAX_CONV 8

typedef struct w2v2_model w2v2_model; /* opaque; owned by the library */

typedef enum {
  W2V2_OK = 0,
  W2V2_E_ARG = 1,     /* null pointer, size or value out of range in a call */
  W2V2_E_CONFIG = 2,  /* inconsistent or unsupported configuration */
  W2V2_E_WEIGHTS = 3, /* weight table: empty, missing/unknown/duplicate name, wrong shape, non-finite value */
  W2V2_E_NOMEM = 4,   /* device memory could not be allocated */
  W2V2_E_DEVICE = 5   /* no such device, not gfx950, or a HIP runtime / launch error */
} w2v2_status;

typedef enum { W2V2_NORM_GROUP = 0, W2V2_NORM_LAYER = 1 } w2v2_feat_norm;
typedef enum { W2V2_FP32 = 0, W2V2_FP16 = 1, W2V2_FP8 = 2, W2V2_FP8_ON_FP32 = 3 } w2v2_precision;
typedef enum { W2V2_GELU_ERF = 0, W2V2_GELU_TANH = 1 } w2v2_gelu;

/*
 * Network shape and workload limits.  The fields mirror the checkpoint config
 * fields the [LiteRT] "Recipe" reads (CTC head width, layer count, feature
 * norm kind, stable layer norm) plus the layouts of [TRT] "Wav2Vec2 CTC
 * layouts".
 *
 *  n_conv, conv_dim/kernel/stride  feature-encoder convs; conv 0 has one input
 *                                  channel.  Unpadded, strided.
 *  conv_bias       1: every conv has a bias.
 *  feat_norm       W2V2_NORM_GROUP: GroupNorm with one group per channel over
 *                  all frames of the window after conv 0 only.
 *                  W2V2_NORM_LAYER: LayerNorm over channels per frame after
 *                  every conv.  Each norm is followed by exact GELU; in the
 *                  group variant convs 1.. are followed by GELU alone.
 *  hidden, heads   model width d and attention heads (d / heads = 16, 32, 64
 *                  or 128).
 *  ffn, layers     feed-forward width and number of transformer blocks.
 *  pos_kernel, pos_groups  positional conv taps K and groups G; padded by
 *                  K/2 on both sides, the last frame dropped for even K.
 *  stable_layer_norm  0: post-norm blocks with the encoder norm before them;
 *                  1: pre-norm blocks with the encoder norm after them.
 *  vocab, blank_id CTC head width and blank token.
 *  eps             epsilon of every GroupNorm / LayerNorm (> 0).
 *  precision       W2V2_FP32: everything in fp32.  W2V2_FP16: fp16 weights
 *                  and matrix operands with fp32 accumulation; residual
 *                  stream, norm statistics, softmax and logits in fp32
 *                  ([TRT] "FP8 quantization study", fp16 graph).
 *                  W2V2_FP8: the fp16 mode with the q/k/v/out/fc1/fc2
 *                  projections of every block on FP8 e4m3 operands ([TRT]
 *                  "FP8 quantization study", "Recipe that was measured"):
 *                  per-tensor weight scales amax(|W|) / 448 taken at create,
 *                  static per-tensor activation scales input_amax / 448 from
 *                  the weight table (see w2v2_calibrate), values beyond
 *                  +-448 saturating, fp32 accumulation, bias after the
 *                  scaling.  Convs, feature projection, positional conv,
 *                  norms, attention and CTC head stay as in the fp16 mode.
 *                  W2V2_FP8_ON_FP32: the same FP8 projections with everything
 *                  else in fp32 ([TRT] "FP8 quantization study": FP8 in the
 *                  fp32 graph).  Both need hidden and ffn to be multiples of
 *                  128.
 *  max_batch       largest batch a forward call may pass (workspace size).
 *  window          samples per PCM window (fixed per model, [LiteRT]
 *                  "Rewrites for the GPU").
 *  gelu_kind       W2V2_GELU_ERF: exact GELU x/2 (1 + erf(x / sqrt 2)) at every
 *                  GELU of the network (default).  W2V2_GELU_TANH: the tanh
 *                  approximation x/2 (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3)))
 *                  everywhere, for parity with graphs exported that way
 *                  ([LiteRT] "Rewrites for the GPU": GELU -> tanh-GELU).
 *
 * Supported limits (else W2V2_E_CONFIG): sample_rate 16000 (the rate the
 * networks of [LiteRT] "Recipe" and [TRT] intro take, with no resampling),
 * 1 <= n_conv <= 8, every conv_dim a
 * multiple of 8 in [8, 2048] with conv_dim[0] <= 512, conv_kernel[0] <= 16,
 * conv_stride[0] <= 8, hidden and ffn multiples of 8, hidden <= 2048,
 * (hidden / pos_groups) a multiple of 8, window long enough for >= 1 frame,
 * at most 16384 frames per window, 1 <= max_batch <= 4096.
 */
typedef struct {
  int32_t abi_version; /* must be W2V2_ABI_VERSION */
  int32_t sample_rate; /* Hz of the PCM; must be 16000 (no resampling is done) */
  int32_t n_conv;
  int32_t conv_dim[W2V2_MAX_CONV];
  int32_t conv_kernel[W2V2_MAX_CONV];
  int32_t conv_stride[W2V2_MAX_CONV];
  int32_t conv_bias;
  int32_t feat_norm;
  int32_t hidden;
  int32_t heads;
  int32_t ffn;
  int32_t layers;
  int32_t pos_kernel;
  int32_t pos_groups;
  int32_t stable_layer_norm;
  int32_t vocab;
  int32_t blank_id;
  float eps;
  int32_t precision;
  int32_t max_batch;
  int32_t window;
  int32_t gelu_kind;
} w2v2_config;

/*
 * One host fp32 weight tensor, row-major and contiguous.  Names and shapes
 * (PyTorch conventions: conv kernels [C_out, C_in / groups, K], linears
 * [out, in]):
 *   fe.conv{i}.weight [C_i, C_{i-1}, k_i] (C_{-1} = 1)   fe.conv{i}.bias [C_i] (if conv_bias)
 *   fe.norm{i}.weight / .bias [C_i]   (i = 0 only in the group variant)
 *   fp.norm.weight / .bias [C_last]   fp.proj.weight [d, C_last]   fp.proj.bias [d]
 *   pos.weight_v [d, d/G, K]  pos.weight_g [K]  pos.bias [d]
 *       (weight norm: one gain per tap, w[:, :, k] = g[k] v[:, :, k] / ||v[:, :, k]||_F)
 *   enc.norm.weight / .bias [d]
 *   layer{l}.attn.{q,k,v,out}.weight [d, d]   layer{l}.attn.{q,k,v,out}.bias [d]
 *   layer{l}.attn_norm.weight / .bias [d]
 *   layer{l}.ffn.fc1.weight [ffn, d]  .fc1.bias [ffn]  .fc2.weight [d, ffn]  .fc2.bias [d]
 *   layer{l}.ffn_norm.weight / .bias [d]
 *   head.weight [vocab, d]  head.bias [vocab]
 * fp8 modes only, one positive value each (shape [1]): the calibrated max |x|
 * of each quantized projection's input,
 *   layer{l}.attn.qkv.input_amax (the input shared by q, k and v)
 *   layer{l}.attn.out.input_amax  layer{l}.ffn.fc1.input_amax  layer{l}.ffn.fc2.input_amax
 * ndim is the number of used entries of shape (1..4).  A shape of [1,1,K]
 * is accepted for pos.weight_g.
 */
typedef struct {
  const char* name;
  const float* data; /* host */
  int32_t ndim;
  int64_t shape[4];
} w2v2_tensor;

/*
 * Build a model on HIP device `device`.
 * Validates the config and the weight table (exactly the names above, each
 * once, with matching shapes and finite values), selects the device, folds
 * the positional-conv weight norm ([LiteRT] "Rewrites for the GPU": folded
 * into a static weight once, not recomputed per call), casts weights to the
 * compute precision, repacks them for the kernels, uploads them and
 * allocates the workspace for max_batch windows.  The weight table is only
 * read during the call; the caller may free it afterwards.
 * On success *out receives the model (free with w2v2_destroy).
 * Errors: W2V2_E_ARG (null cfg/out, n_weights < 0), W2V2_E_CONFIG,
 * W2V2_E_WEIGHTS, W2V2_E_DEVICE (no such device / not gfx950),
 * W2V2_E_NOMEM.  On error *out is set to NULL and nothing is leaked.
 */
w2v2_status w2v2_create(const w2v2_config* cfg, const w2v2_tensor* weights, int32_t n_weights,
                        int32_t device, w2v2_model** out);

/* Release the model's device memory.  NULL is a no-op.  The caller must have
 * synchronized every stream that still uses the model. */
void w2v2_destroy(w2v2_model* model);

/*
 * Frames the feature encoder produces from `samples` input samples: the
 * unpadded conv length rule floor((L - k) / s) + 1 (0 if L < k) applied
 * conv by conv.  With samples = the valid length of a row this is the
 * number of frames to decode ([LiteRT] "Rewrites for the GPU").  Host only.
 * Errors: W2V2_E_ARG (null pointer, samples < 0).
 */
w2v2_status w2v2_num_frames(const w2v2_model* model, int64_t samples, int32_t* frames);

/* Frames per window T, vocab V and workspace bytes of a model (host only;
 * any output pointer may be NULL). */
w2v2_status w2v2_model_info(const w2v2_model* model, int32_t* frames_per_window, int32_t* vocab,
                            int64_t* workspace_bytes);

/*
 * Whole network on one batch of windows.
 *   pcm     dev fp32 [batch, window]: raw 16 kHz samples.  Samples at or after
 *           valid[b] are treated as 0 whatever the buffer holds (zero-padded
 *           window, [LiteRT] "Rewrites for the GPU").
 *   valid   dev int32 [batch]: valid samples per row, 0 <= valid[b] <= window
 *           (the device clamps out-of-range values into that range).
 *   batch   1 <= batch <= max_batch.
 *   logits  dev fp32 [batch, T, vocab]: CTC logits for every frame of the
 *           window (T = frames per window); attention runs over all T frames
 *           with no mask.
 *   vframes dev int32 [batch] or NULL: frames to decode per row
 *           (w2v2_num_frames of valid[b], computed on the device).
 * Execution: for batch >= 2 the two halves of the batch run concurrently,
 * the first on `stream`, the second on a stream the model owns that is
 * forked from and joined back to `stream` with events, so the call remains
 * asynchronous and ordered on `stream`.  Results are bit-identical to a
 * serial run (rows are independent).  While w2v2_profile_enable profiles
 * every kernel (no filter), the whole batch runs as one pass on `stream`.
 * Errors: W2V2_E_ARG (null model/pcm/valid/logits, batch out of range),
 * W2V2_E_DEVICE (launch failure).
 */
w2v2_status w2v2_forward(w2v2_model* model, const float* pcm, const int32_t* valid, int32_t batch,
                         float* logits, int32_t* vframes, void* stream);

/*
 * Whole network plus greedy CTC decoding in one call: w2v2_forward followed
 * by the decoding of w2v2_ctc_greedy ([TRT] "Method": per-frame argmax, CTC
 * token ids), with the per-frame argmax taken inside the CTC head's GEMM
 * epilogue from the fp32 values it stores, so the logits are not read back.
 *   pcm, valid, batch, logits  as in w2v2_forward (logits are still written).
 *   vframes  dev int32 [batch]: frames decoded per row (required).
 *   ids      dev int32 [batch, T]: ids[b, 0 .. lens[b]) are the tokens of row
 *            b (runs of equal per-frame argmax merged, blank_id dropped), the
 *            rest -1.
 *   lens     dev int32 [batch].
 * The argmax takes the lowest index on ties (-0 and +0 are equal), so ids and
 * lens are bit-identical to w2v2_ctc_greedy applied to the logits.  Same
 * execution and stream rules as w2v2_forward; allocates nothing.
 * Errors: as w2v2_forward, plus W2V2_E_ARG if vframes, ids or lens is NULL.
 */
w2v2_status w2v2_forward_greedy(w2v2_model* model, const float* pcm, const int32_t* valid, int32_t batch,
                                float* logits, int32_t* vframes, int32_t* ids, int32_t* lens, void* stream);

/*
 * w2v2_forward_greedy for callers that cannot allocate device memory or
 * should not touch the model's workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Identical results
 * (bitwise) to w2v2_forward_greedy, but every intermediate buffer (conv
 * outputs, GroupNorm partials, residual stream, GEMM operands, argmax keys)
 * lives in one static device array of the library, 64 MiB, that each GPU the
 * library runs on holds until the process ends; the call allocates nothing.
 * Limit: the batch's intermediates must fit in 64 MiB (about 10 one-second
 * windows of the base network, none of a 16 s one); larger batches are
 * rejected with W2V2_E_ARG before any device work.  Every call on a GPU
 * shares that GPU's array (whatever the model), so calls that overlap on one
 * GPU race: serialize them.
 * Arguments, stream rules and errors as w2v2_forward_greedy.
 */
w2v2_status w2v2_forward_greedy_noalloc(w2v2_model* model, const float* pcm, const int32_t* valid,
                                        int32_t batch, float* logits, int32_t* vframes, int32_t* ids,
                                        int32_t* lens, void* stream);

/*
 * Static activation calibration of the fp8 mode ([TRT] "Recipe that was
 * measured": max(abs(input)) of every quantized projection, recorded on the
 * float model over calibration clips).  Runs w2v2_forward on the batch with a
 * W2V2_FP32 or W2V2_FP16 model and raises
 *   amax  dev fp32 [layers][4]: slot [l][k] = max over the batch (and over
 *         earlier calls: the caller zero-fills it once, then calls this for
 *         each calibration batch) of |x| at the input of layer l's
 *         k = 0 q/k/v, 1 out, 2 fc1, 3 fc2 projection.
 * The values written to `logits` are w2v2_forward's.  The entries
 * layer{l}.<input>.input_amax of a model in an fp8 mode are these values.
 * Errors: W2V2_E_ARG (null model / amax, or a model in an fp8 mode), and as
 * w2v2_forward.
 */
w2v2_status w2v2_calibrate(w2v2_model* model, const float* pcm, const int32_t* valid, int32_t batch,
                           float* logits, float* amax, void* stream);

/*
 * Whole network with every row taken as its own true-length clip ([TRT]
 * "Wav2Vec2 CTC layouts": true-length PCM input, no padded-batch attention
 * mask): row b is computed exactly as a single clip of its first valid[b]
 * samples, so its conv layers, the group norm over time of conv 0, the
 * positional conv's zero padding and the attention cover only that clip's
 * frames.  The rows are packed inside the library, so the work scales with
 * the valid audio rather than with batch x window.
 *   pcm        dev fp32 [batch, window]; only the first valid[b] samples of
 *              row b are read.
 *   valid_host HOST int32 [batch]: valid samples per row, 0 <= valid[b] <=
 *              window.  Read during the call (launch sizes depend on it); the
 *              caller may reuse the array as soon as the call returns.
 *   batch      1 <= batch <= max_batch.
 *   logits     dev fp32 [batch, T, vocab] (T = frames per window): frame t of
 *              row b for t < w2v2_num_frames(valid[b]), 0 for later frames.
 *   vframes    dev int32 [batch] or NULL: w2v2_num_frames(valid[b]).
 * Asynchronous on `stream` like w2v2_forward: the lengths are copied into a
 * pinned staging buffer that w2v2_create allocated and uploaded on that
 * stream; a call first waits for the previous call's upload from that buffer.
 * As in w2v2_forward, for batch >= 2 the two halves of the rows run
 * concurrently (each packed on its own), the second on the model's stream
 * forked after the upload and joined back; profiling every kernel runs one
 * pass.  Results are bit-identical to one pass.
 * Allocates nothing.  Calls that share a model must not overlap.
 * Errors: W2V2_E_ARG (null model/pcm/valid_host/logits, batch out of range,
 * a valid[b] outside [0, window]), W2V2_E_DEVICE (copy or launch failure).
 */
w2v2_status w2v2_forward_true_length(w2v2_model* model, const float* pcm, const int32_t* valid_host,
                                     int32_t batch, float* logits, int32_t* vframes, void* stream);

/*
 * Feature-encoder stage only (conv 0 .. conv n-1 with their norms and GELU):
 *   features dev fp32 [batch, T, C_last] (channels-last).
 * Same pcm / valid / batch rules as w2v2_forward.  Together with
 * w2v2_forward_encoder it splits w2v2_forward at the conv-frontend /
 * encoder boundary ([LiteRT] "Rewrites for the GPU", two-graph split), for
 * stage timing and stage-level checks; w2v2_forward itself does not pass
 * through fp32 features.
 */
w2v2_status w2v2_forward_frontend(w2v2_model* model, const float* pcm, const int32_t* valid,
                                  int32_t batch, float* features, void* stream);

/*
 * Encoder stage only: feature projection, positional conv, blocks, CTC head.
 *   features dev fp32 [batch, T, C_last]; logits dev fp32 [batch, T, vocab].
 * Errors as w2v2_forward.
 */
w2v2_status w2v2_forward_encoder(w2v2_model* model, const float* features, int32_t batch,
                                 float* logits, void* stream);

/*
 * Greedy CTC decoding ([TRT] "Method": per-frame argmax and CTC token ids).
 * For each row b: a[t] = argmax_v logits[b, t, v] (lowest index on ties) for
 * t < vframes[b]; the path is collapsed by merging runs of equal ids and
 * dropping blank_id.
 *   logits  dev fp32 [batch, frames, vocab]   vframes dev int32 [batch]
 *           (values are clamped into [0, frames])
 *   ids     dev int32 [batch, frames]: ids[b, 0 .. lens[b]) are the tokens,
 *           the rest is -1.  Also used as scratch for the argmax path.
 *   lens    dev int32 [batch].
 * Needs no model; independent of w2v2_forward so that it can be fed any
 * logits (for example one-hot logits of a hand-written path).
 * Errors: W2V2_E_ARG (null pointer, batch < 1, frames < 1 or > 16384,
 * vocab < 1, blank_id outside [0, vocab)), W2V2_E_DEVICE.
 */
w2v2_status w2v2_ctc_greedy(const float* logits, const int32_t* vframes, int32_t batch,
                            int32_t frames, int32_t vocab, int32_t blank_id, int32_t* ids,
                            int32_t* lens, void* stream);

/*
 * Per-kernel timing with HIP events.  When enabled, the model's calls record
 * an event pair around every kernel they launch (on the stream the kernel
 * runs on), or, if `only` is not NULL, around the launches whose kernel name
 * equals `only` (so a timed loop can watch one kernel with two events per
 * launch).  Without `only`, w2v2_forward runs the whole batch as one pass
 * on the caller's stream, so every timed kernel runs alone; with `only` it
 * keeps the two halves concurrent, and a timed launch then shares the GPU
 * with the other half's kernels.  `only` = "stage" times no kernel but
 * records, for every part of the batch that w2v2_forward / w2v2_forward_greedy
 * runs (the two concurrent halves), one pair around its conv frontend
 * ("stage_frontend") and one around its encoder and CTC head
 * ("stage_encoder") on the part's stream: the frontend / encoder boundary of
 * the unchanged concurrent execution ([LiteRT] "Rewrites for the GPU",
 * two-graph split).
 * w2v2_profile_read synchronizes on the recorded events, accumulates the
 * per-kernel-name totals since the last read, and writes up to `cap`
 * entries: names[i] (static strings owned by the library), total_ms[i] and
 * launches[i].  *n receives the number of distinct kernel names.
 * Errors: W2V2_E_ARG, W2V2_E_DEVICE.
 */
w2v2_status w2v2_profile_enable(w2v2_model* model, int32_t enable, const char* only);
w2v2_status w2v2_profile_read(w2v2_model* model, int32_t cap, const char** names, double* total_ms,
                              int64_t* launches, int32_t* n);

/* Message of the last failing call on this thread ("" if none). */
const char* w2v2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W2V2_H */
