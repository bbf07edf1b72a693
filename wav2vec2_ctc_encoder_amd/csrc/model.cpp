// Runtime and C ABI of the wav2vec2-CTC inference library.
//
// w2v2_create validates the configuration and the weight table, folds the
// positional-conv weight norm (w = g * v / ||v|| per tap, in double), casts
// the weights to the operand type, repacks them into the layouts the
// kernels read (conv kernels as [C_out, k*C_in] GEMM rows, fused QKV, the
// positional conv split per group) and uploads them as one allocation.  The
// workspace for max_batch windows is allocated once; the forward calls only
// enqueue kernels on the caller's stream.
//
// Data layout in device memory (channels-last throughout):
//   conv i output        [B, T_i, C_i]   operand type, ping-pong buffers A/B
//   GroupNorm partials   [B, chunks, k + k(k+1)/2] fp64 (input lag statistics)
//   residual stream h    [B*T, d]        fp32 (post-norm: the raw residual sum,
//                                        normalised by its reader; see run_encoder)
//   LayerNorm row stats  [B*T] (mean, rstd) fp32
//   GEMM operand x       [B*T, max(d, C_last)]  operand type (LayerNorm output)
//   qkv                  [B*T, 3d]       operand type
//   attention out        [B*T, d]        operand type
//   FFN hidden           [B*T, ffn]      operand type
//   pos-conv input       [G][B][T + K][d/G] operand type, zero padded
//   true-length tables   per-level row lengths / packed starts (int32), the
//                        table bases (int64) and the per-row offset tables
//                        of the conv / positional-conv A operands and the
//                        head's output rows (int64)
//
// True-length mode (w2v2_forward_true_length): every row is computed as its
// own clip of valid[b] samples.  Rows are packed per level (row b's frames of
// conv i at packed rows start_i[b] .. start_i[b] + len_i[b] - 1), so the conv
// GEMMs, the encoder GEMMs and the row kernels run over the packed rows only;
// the strided conv windows, the positional conv's padded input and the head's
// [B, T, V] output rows are reached through the per-row offset tables.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/w2v2.h"
#include "common.h"

using namespace w2v2;

namespace {

thread_local std::string g_last_error;

w2v2_status fail(w2v2_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) (void)hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

int conv_len(int64_t n, int k, int s) { return n < k ? 0 : (int)((n - k) / s + 1); }

// Inputs of the fp8 mode's projections, in the order of their calibration
// slots: q/k/v (one shared input), out, fc1, fc2.
const char* const kFp8Inputs[4] = {"attn.qkv", "attn.out", "ffn.fc1", "ffn.fc2"};

struct ExpectedW {
  std::string name;
  std::vector<int64_t> shape;
};

std::vector<ExpectedW> expected_weights(const w2v2_config& c) {
  std::vector<ExpectedW> out;
  int64_t cin = 1;
  for (int i = 0; i < c.n_conv; ++i) {
    const int64_t ci = c.conv_dim[i];
    out.push_back({"fe.conv" + std::to_string(i) + ".weight", {ci, cin, c.conv_kernel[i]}});
    if (c.conv_bias) out.push_back({"fe.conv" + std::to_string(i) + ".bias", {ci}});
    if (c.feat_norm == W2V2_NORM_LAYER || i == 0) {
      out.push_back({"fe.norm" + std::to_string(i) + ".weight", {ci}});
      out.push_back({"fe.norm" + std::to_string(i) + ".bias", {ci}});
    }
    cin = ci;
  }
  const int64_t d = c.hidden, cl = c.conv_dim[c.n_conv - 1];
  out.push_back({"fp.norm.weight", {cl}});
  out.push_back({"fp.norm.bias", {cl}});
  out.push_back({"fp.proj.weight", {d, cl}});
  out.push_back({"fp.proj.bias", {d}});
  out.push_back({"pos.weight_v", {d, d / c.pos_groups, c.pos_kernel}});
  out.push_back({"pos.weight_g", {c.pos_kernel}});
  out.push_back({"pos.bias", {d}});
  out.push_back({"enc.norm.weight", {d}});
  out.push_back({"enc.norm.bias", {d}});
  for (int l = 0; l < c.layers; ++l) {
    const std::string p = "layer" + std::to_string(l) + ".";
    for (const char* pr : {"q", "k", "v", "out"}) {
      out.push_back({p + "attn." + pr + ".weight", {d, d}});
      out.push_back({p + "attn." + pr + ".bias", {d}});
    }
    out.push_back({p + "attn_norm.weight", {d}});
    out.push_back({p + "attn_norm.bias", {d}});
    out.push_back({p + "ffn.fc1.weight", {c.ffn, d}});
    out.push_back({p + "ffn.fc1.bias", {c.ffn}});
    out.push_back({p + "ffn.fc2.weight", {d, c.ffn}});
    out.push_back({p + "ffn.fc2.bias", {d}});
    out.push_back({p + "ffn_norm.weight", {d}});
    out.push_back({p + "ffn_norm.bias", {d}});
    if (c.precision == W2V2_FP8 || c.precision == W2V2_FP8_ON_FP32)
      for (const char* w : kFp8Inputs) out.push_back({p + w + ".input_amax", {1}});
  }
  out.push_back({"head.weight", {c.vocab, d}});
  out.push_back({"head.bias", {c.vocab}});
  return out;
}

std::string check_config(const w2v2_config& c, int* frames_out) {
  auto bad = [](const char* m) { return std::string(m); };
  if (c.abi_version != W2V2_ABI_VERSION) return bad("abi_version does not match W2V2_ABI_VERSION");
  if (c.sample_rate != 16000) return bad("sample_rate must be 16000 (PCM is not resampled)");
  if (c.n_conv < 1 || c.n_conv > W2V2_MAX_CONV) return bad("n_conv must be in [1, 8]");
  for (int i = 0; i < c.n_conv; ++i) {
    if (c.conv_dim[i] < 8 || c.conv_dim[i] > 2048 || c.conv_dim[i] % 8)
      return bad("conv_dim must be a multiple of 8 in [8, 2048]");
    if (c.conv_kernel[i] < 1 || c.conv_stride[i] < 1) return bad("conv kernel and stride must be >= 1");
  }
  if (c.conv_dim[0] > 512) return bad("conv_dim[0] must be <= 512");
  if (c.conv_kernel[0] > 16) return bad("conv_kernel[0] must be <= 16");
  if (c.conv_stride[0] > 8) return bad("conv_stride[0] must be <= 8");
  if (c.conv_bias != 0 && c.conv_bias != 1) return bad("conv_bias must be 0 or 1");
  if (c.feat_norm != W2V2_NORM_GROUP && c.feat_norm != W2V2_NORM_LAYER) return bad("unknown feat_norm");
  if (c.hidden < 8 || c.hidden > 2048 || c.hidden % 8) return bad("hidden must be a multiple of 8 in [8, 2048]");
  if (c.heads < 1 || c.hidden % c.heads) return bad("hidden must be divisible by heads");
  if (!attention_supported(c.hidden / c.heads)) return bad("head size hidden/heads must be 16, 32, 64 or 128");
  if (c.ffn < 8 || c.ffn % 8) return bad("ffn must be a positive multiple of 8");
  if (c.layers < 0) return bad("layers must be >= 0");
  if (c.pos_kernel < 1 || c.pos_groups < 1) return bad("pos_kernel and pos_groups must be >= 1");
  if (c.hidden % c.pos_groups || (c.hidden / c.pos_groups) % 8)
    return bad("hidden / pos_groups must be a multiple of 8");
  if (c.stable_layer_norm != 0 && c.stable_layer_norm != 1) return bad("stable_layer_norm must be 0 or 1");
  if (c.vocab < 1) return bad("vocab must be >= 1");
  if (c.blank_id < 0 || c.blank_id >= c.vocab) return bad("blank_id must be in [0, vocab)");
  if (!(c.eps > 0.f) || !std::isfinite(c.eps)) return bad("eps must be positive and finite");
  if (c.precision != W2V2_FP32 && c.precision != W2V2_FP16 && c.precision != W2V2_FP8 &&
      c.precision != W2V2_FP8_ON_FP32)
    return bad("unknown precision");
  const bool fp8 = c.precision == W2V2_FP8 || c.precision == W2V2_FP8_ON_FP32;
  if (fp8 && (c.hidden % 128 || c.ffn % 128))
    return bad("the fp8 mode needs hidden and ffn to be multiples of 128");
  if (c.gelu_kind != W2V2_GELU_ERF && c.gelu_kind != W2V2_GELU_TANH) return bad("unknown gelu_kind");
  if (c.max_batch < 1 || c.max_batch > 4096) return bad("max_batch must be in [1, 4096]");
  if (c.window < 1) return bad("window must be >= 1");
  int64_t n = c.window;
  for (int i = 0; i < c.n_conv; ++i) n = conv_len(n, c.conv_kernel[i], c.conv_stride[i]);
  if (n < 1) return bad("window is shorter than the feature encoder's receptive field");
  if (n > 16384) return bad("at most 16384 frames per window are supported");
  const int64_t t0 = conv_len(c.window, c.conv_kernel[0], c.conv_stride[0]);
  if ((int64_t)c.max_batch * t0 > (int64_t)INT32_MAX / 2) return bad("max_batch * frames of conv 0 too large");
  *frames_out = (int)n;
  return "";
}

// ----------------------------------------------------------------------------
// kernel timing
// ----------------------------------------------------------------------------
struct Profiler : LaunchHook {
  struct Rec {
    const char* name;
    hipEvent_t a, b;
  };
  std::vector<hipEvent_t> pool;
  std::vector<Rec> recs;
  std::map<std::string, std::pair<double, int64_t>> totals;
  std::map<std::string, const char*> names;  // stable name strings
  hipEvent_t pending = nullptr;
  hipError_t err = hipSuccess;

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) err = r;
    return e;
  }
  void before(const char*, hipStream_t s) override {
    pending = get();
    if (pending) {
      hipError_t r = hipEventRecord(pending, s);
      if (r != hipSuccess) err = r;
    }
  }
  void after(const char* name, hipStream_t s) override {
    hipEvent_t e = get();
    if (e) {
      hipError_t r = hipEventRecord(e, s);
      if (r != hipSuccess) err = r;
    }
    if (pending && e) recs.push_back({name, pending, e});
    pending = nullptr;
  }
  ~Profiler() override {
    for (auto& r : recs) {
      (void)hipEventDestroy(r.a);
      (void)hipEventDestroy(r.b);
    }
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};

}  // namespace

// ----------------------------------------------------------------------------
// model
// ----------------------------------------------------------------------------
// Workspace regions of one forward (the whole batch, or one half of it).
struct Ws {
  void *bufA = nullptr, *bufB = nullptr;
  double* gn_part = nullptr;
  float2* gn_ss = nullptr;
  float* h = nullptr;
  void *x = nullptr, *qkv = nullptr, *attn = nullptr, *ffn = nullptr, *zg = nullptr;
  float2* lnst = nullptr;  // (mean, rstd) per row of the last post-norm LayerNorm
  uint64_t* keys = nullptr;  // per-frame argmax keys of the CTC head (w2v2_forward_greedy)
  bool shared = false;     // another part of the batch runs concurrently
};
constexpr int kWsRegions = 12;
// w2v2_forward splits a batch into up to kSplit row ranges that run
// concurrently, one per stream (the caller's and kSplit - 1 of the model's).
constexpr int kSplit = 2;

struct w2v2_model {
  w2v2_config cfg{};
  int device = 0;
  DType dt = DType::F16;
  int act = 1;                // GELU code of the kernels: 1 erf, 2 tanh
  int T[W2V2_MAX_CONV] = {};  // frames after conv i
  int Tf = 0;                 // frames per window

  void* wmem = nullptr;
  size_t wbytes = 0;
  void* ws = nullptr;
  size_t wsbytes = 0;

  // weights (device)
  struct Conv {
    const void* w = nullptr;      // i = 0: fp32 [C][k]; i > 0: operand type [C_out][k*C_in]
    const float* bias = nullptr;  // fp32 [C] or null
    const float* gamma = nullptr;
    const float* beta = nullptr;
  } conv[W2V2_MAX_CONV];
  const float *fp_g = nullptr, *fp_b = nullptr, *fp_bias = nullptr;
  const void* fp_w = nullptr;
  const void* pos_w = nullptr;  // [G][Cg][K*Cg]
  const float* pos_bias = nullptr;
  const float *enc_g = nullptr, *enc_b = nullptr;
  struct Layer {
    const void *wqkv = nullptr, *wo = nullptr, *w1 = nullptr, *w2 = nullptr;
    const float *bqkv = nullptr, *bo = nullptr, *b1 = nullptr, *b2 = nullptr;
    const float *ln1_g = nullptr, *ln1_b = nullptr, *ln2_g = nullptr, *ln2_b = nullptr;
    // fp8 mode: per-column accumulator scales (activation scale x weight
    // scale) of the qkv / out / fc1 / fc2 GEMMs and the inverse activation
    // scales 448 / amax of their inputs, in that order
    const float* cs[4] = {};
    float inv[4] = {1.f, 1.f, 1.f, 1.f};
  };
  std::vector<Layer> layers;
  const void* head_w = nullptr;
  const float* head_b = nullptr;

  // workspace regions; row_bytes[i] is region i's share per batch row (in
  // Ws field order), so rows [b0, b0 + n) of every region form a Ws of
  // their own.  The positional-conv input [G][n][T + K][d/G] of such a
  // slice is contiguous inside its share.
  Ws w;
  size_t row_bytes[kWsRegions] = {};
  // the model's own streams of w2v2_forward (parts 1 .. kSplit-1 of the
  // batch run there) and the events that fork them from and join them back
  // to the caller's stream
  hipStream_t aux[kSplit] = {};
  hipEvent_t ev_fork = nullptr, ev_join[kSplit] = {};
  int32_t* tl_i32 = nullptr;  // true-length: [2 * n_conv + 1][max_batch] lengths, starts, valid
  int64_t* tl_base = nullptr; // [n_conv + 1][max_batch] table bases
  int64_t* tl_rows = nullptr; // per-row offset tables
  int64_t* tl_pinned = nullptr;  // pinned host staging of the int32 + int64 part
  size_t tl_bytes = 0;
  hipEvent_t tl_copied = nullptr; // recorded after each upload from tl_pinned
  bool tl_pending = false;

  Profiler* prof = nullptr;
  bool prof_on = false;
  bool fp8 = false;           // fp8 mode: e4m3 encoder projections
  void* scratch = nullptr;    // this device's static scratch (w2v2_forward_greedy_noalloc)
  float* calib = nullptr;     // during w2v2_calibrate: [layers][4] amax slots
  std::string prof_only;  // empty: every kernel

  ~w2v2_model() {
    delete prof;
    if (ev_fork) (void)hipEventDestroy(ev_fork);
    for (int i = 0; i < kSplit; ++i) {
      if (ev_join[i]) (void)hipEventDestroy(ev_join[i]);
      if (aux[i]) (void)hipStreamDestroy(aux[i]);
    }
    if (tl_copied) (void)hipEventDestroy(tl_copied);
    if (tl_pinned) (void)hipHostFree(tl_pinned);
    if (wmem) (void)hipFree(wmem);
    if (ws) (void)hipFree(ws);
  }
};

namespace {

struct Arena {
  std::vector<uint8_t> bytes;
  size_t add(const void* src, size_t n) {
    size_t off = (bytes.size() + 255) & ~size_t(255);
    bytes.resize(off + n);
    memcpy(bytes.data() + off, src, n);
    return off;
  }
};

size_t add_f32(Arena& a, const std::vector<float>& v) { return a.add(v.data(), v.size() * 4); }

// e4m3 (OCP FP8: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits) code
// of v: the nearest of +-2^E (1 + m/8), E = -6 .. 8 (448 the largest), and
// the subnormals +-2^-6 m/8, ties to the even mantissa; larger magnitudes
// saturate to 448.  Weights are quantized with it at create.
uint8_t e4m3_code(double v) {
  const uint8_t sign = std::signbit(v) ? 0x80 : 0;
  const double a = std::fabs(v);
  if (!(a == a)) return 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  int e = 0;
  std::frexp(a, &e);                                 // a = f 2^e, f in [0.5, 1)
  int E = std::max(e - 1, -6);
  const double q = std::ldexp(1.0, E - 3);           // grid spacing of a's binade
  const double r = std::nearbyint(a / q) * q;        // round to nearest, ties to even
  if (r >= 448.0) return sign | 0x7E;
  if (r == 0.0) return sign;
  std::frexp(r, &e);
  E = e - 1;
  if (E < -6) return sign | (uint8_t)std::lrint(r / std::ldexp(1.0, -9));   // subnormal: m = r / 2^-9
  const int mant = (int)std::lrint((r / std::ldexp(1.0, E) - 1.0) * 8.0);
  return sign | (uint8_t)(((E + 7) << 3) | mant);
}

double amax_of(const float* p, size_t n) {
  double mx = 0.0;
  for (size_t i = 0; i < n; ++i) mx = std::max(mx, (double)std::fabs(p[i]));
  return mx;
}

// v as e4m3 codes, consecutive blocks of `block` values with their own scales
// (the per-tensor weight scales amax / 448; a zero tensor keeps scale 0 and
// codes 0)
size_t add_e4m3(Arena& a, const std::vector<float>& v, const std::vector<double>& scale, size_t block) {
  std::vector<uint8_t> q(v.size());
  for (size_t i = 0; i < v.size(); ++i) {
    const double sc = scale[i / block];
    q[i] = sc > 0.0 ? e4m3_code((double)v[i] / sc) : 0;
  }
  return a.add(q.data(), q.size());
}


// one fp8 linear [N, K]: the e4m3 weight and its per-column accumulator
// scales (input amax / 448) x (weight amax / 448)
size_t add_fp8_linear(Arena& a, const std::vector<float>& w, double in_amax, int N, size_t* cs_off) {
  const double sw = amax_of(w.data(), w.size()) / 448.0;
  const size_t off = add_e4m3(a, w, {sw}, w.size());
  *cs_off = add_f32(a, std::vector<float>((size_t)N, (float)(in_amax / 448.0 * sw)));
  return off;
}

size_t add_t(Arena& a, DType dt, const std::vector<float>& v) {
  if (dt == DType::F32) return add_f32(a, v);
  std::vector<_Float16> h(v.size());
  for (size_t i = 0; i < v.size(); ++i) h[i] = (_Float16)v[i];
  return a.add(h.data(), h.size() * 2);
}

#define W2V2_LAUNCH(m, s, name, call)                                                 \
  do {                                                                                \
    const bool p_ = (m)->prof_on && ((m)->prof_only.empty() || (m)->prof_only == name); \
    if (p_) (m)->prof->before(name, s);                                               \
    hipError_t e_ = (call);                                                           \
    if (p_) (m)->prof->after(name, s);                                                \
    if (e_ != hipSuccess)                                                             \
      return fail(W2V2_E_DEVICE, std::string(name) + ": " + hipGetErrorString(e_));  \
  } while (0)

// int32 words of the true-length length/start/valid block (kept a multiple of 2
// so that the int64 bases behind it stay aligned)
int64_t tl_i32_words(const w2v2_config& c) { return (((int64_t)2 * c.n_conv + 1) * c.max_batch + 1) & ~int64_t(1); }
// entries of the per-row tables: conv 1..n-1 A rows, positional-conv A rows, head output rows
int64_t tl_rows_count(const w2v2_config& c, const int* T, int Tf) {
  int64_t n = 2 * (int64_t)Tf;
  for (int i = 1; i < c.n_conv; ++i) n += T[i];
  return n * c.max_batch;
}

// True-length packing of one forward call (see the header); null: padded windows.
struct Packing {
  int64_t P[W2V2_MAX_CONV] = {};                 // packed rows per conv level
  RowSpan lvl[W2V2_MAX_CONV];                    // per-row frames and starts (device)
  const int64_t* a_rows[W2V2_MAX_CONV] = {};     // conv i >= 1: A row offsets
  const int64_t* pos_rows = nullptr;             // positional-conv A row offsets
  const int64_t* head_rows = nullptr;            // head output row offsets in [B, T, V]
};

// conv 0 .. n-1; returns the final conv output buffer in *feat
w2v2_status run_frontend(w2v2_model* m, const Ws& w, const float* pcm, const int32_t* valid, int B, hipStream_t s,
                         const void** feat, const Packing* pk = nullptr) {
  const w2v2_config& c = m->cfg;
  const DType dt = m->dt;
  const int C0 = c.conv_dim[0];
  const RowSpan rows0 = pk ? pk->lvl[0] : RowSpan{};
  if (c.feat_norm == W2V2_NORM_GROUP) {
    W2V2_LAUNCH(m, s, "gn0_stats",
                launch_gn0_stats(pcm, valid, c.window, B, c.conv_kernel[0], c.conv_stride[0], m->T[0], rows0.len,
                                 w.gn_part, s));
    W2V2_LAUNCH(m, s, "gn0_finalize",
                launch_gn0_finalize(w.gn_part, B, c.conv_kernel[0], m->T[0], rows0.len, (const float*)m->conv[0].w,
                                    m->conv[0].bias, C0, m->conv[0].gamma, m->conv[0].beta, c.eps, w.gn_ss, s));
    W2V2_LAUNCH(m, s, "conv0_gn_gelu",
                launch_conv0(dt, pcm, valid, c.window, B, (const float*)m->conv[0].w, m->conv[0].bias, C0,
                             c.conv_kernel[0], c.conv_stride[0], m->T[0], rows0, w.bufA, w.gn_ss, nullptr,
                             nullptr, c.eps, m->act, s));
  } else {
    W2V2_LAUNCH(m, s, "conv0_ln_gelu",
                launch_conv0(dt, pcm, valid, c.window, B, (const float*)m->conv[0].w, m->conv[0].bias, C0,
                             c.conv_kernel[0], c.conv_stride[0], m->T[0], rows0, w.bufA, nullptr,
                             m->conv[0].gamma, m->conv[0].beta, c.eps, m->act, s));
  }
  const void* cur = w.bufA;
  int tin = m->T[0], cin = C0;
  for (int i = 1; i < c.n_conv; ++i) {
    void* out = (i & 1) ? w.bufB : w.bufA;
    GemmArgs g;
    g.role = kGemmConv;
    g.A = cur;
    g.lda = (int64_t)c.conv_stride[i] * cin;
    g.a_seg = (int64_t)tin * cin;
    g.seg_rows = m->T[i];
    g.a_rows = pk ? pk->a_rows[i] : nullptr;
    g.B = m->conv[i].w;
    g.M = (int)(pk ? pk->P[i] : (int64_t)B * m->T[i]);
    g.N = c.conv_dim[i];
    g.K = c.conv_kernel[i] * cin;
    g.bias = m->conv[i].bias;
    g.out_t = out;
    g.ldc = c.conv_dim[i];
    g.act = (c.feat_norm == W2V2_NORM_GROUP) ? m->act : 0;
    static const char* kConvName[W2V2_MAX_CONV] = {"conv0",      "conv1_gemm", "conv2_gemm", "conv3_gemm",
                                                    "conv4_gemm", "conv5_gemm", "conv6_gemm", "conv7_gemm"};
    W2V2_LAUNCH(m, s, kConvName[i], launch_gemm(dt, g, s));
    if (c.feat_norm == W2V2_NORM_LAYER) {
      W2V2_LAUNCH(m, s, "conv_ln_gelu",
                  launch_layernorm(dt, nullptr, out, g.M, c.conv_dim[i], m->conv[i].gamma,
                                   m->conv[i].beta, c.eps, nullptr, out, m->act, nullptr, s));
    }
    cur = out;
    tin = m->T[i];
    cin = c.conv_dim[i];
  }
  *feat = cur;
  return W2V2_OK;
}

// LayerNorm applied to a GEMM's residual as it is read (post-norm blocks)
struct ResNorm {
  const float2* stats;
  const float *gamma, *beta;
};

// Operands and outputs of an encoder projection beyond the defaults: in the
// fp8 mode e4m3 operands with per-column accumulator scales and optionally
// e4m3 output; during calibration the amax slot of the output.
struct ProjIO {
  bool f8 = false;
  const float* col_scale = nullptr;
  uint8_t* out8 = nullptr;
  float out8_inv = 1.f;
  float* out_amax = nullptr;
};

w2v2_status gemm_linear(w2v2_model* m, hipStream_t s, const char* name, int role, const void* A, int M, int N,
                        int K, const void* W, const float* bias, int act, const float* residual, float* out32,
                        void* outt, int64_t ldc, const ResNorm* rn = nullptr, const ProjIO& io = ProjIO()) {
  GemmArgs g;
  g.role = role;
  g.A = A;
  g.lda = K;
  g.a_seg = 0;
  g.seg_rows = M;
  g.B = W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.bias = bias;
  g.act = act;
  g.residual = residual;
  if (rn) {
    g.res_stats = rn->stats;
    g.res_gamma = rn->gamma;
    g.res_beta = rn->beta;
  }
  g.out_f32 = out32;
  g.out_t = io.out8 ? nullptr : outt;
  g.ldc = ldc;
  g.col_scale = io.col_scale;
  g.out_t_f32 = io.f8 && m->dt == DType::F32;
  g.out_f8 = io.out8;
  g.out_f8_inv = io.out8_inv;
  g.out_amax = io.out_amax;
  W2V2_LAUNCH(m, s, name, launch_gemm(io.f8 ? DType::F8 : m->dt, g, s));
  return W2V2_OK;
}

#define W2V2_TRY(call)                  \
  do {                                  \
    w2v2_status st_ = (call);           \
    if (st_ != W2V2_OK) return st_;     \
  } while (0)

// keys: null, or the argmax slots of the B * T output frames, zero-filled,
// which the head raises to each frame's argmax key.
w2v2_status run_encoder(w2v2_model* m, const Ws& w, const void* feat, int B, float* logits, hipStream_t s,
                        const Packing* pk = nullptr, uint64_t* keys = nullptr) {
  const w2v2_config& c = m->cfg;
  const DType dt = m->dt;
  const int T = m->Tf, d = c.hidden, F = c.ffn, G = c.pos_groups, Cg = d / G, K = c.pos_kernel;
  const int cl = c.conv_dim[c.n_conv - 1];
  const int M = (int)(pk ? pk->P[c.n_conv - 1] : (int64_t)B * T);  // rows of the encoder
  const RowSpan rows = pk ? pk->lvl[c.n_conv - 1] : RowSpan{};
  const float eps = c.eps;

  // feature projection: LN over channels, then Linear C -> d (fp32 residual stream)
  W2V2_LAUNCH(m, s, "layernorm",
              launch_layernorm(dt, nullptr, feat, M, cl, m->fp_g, m->fp_b, eps, nullptr, w.x, 0, nullptr, s));
  W2V2_TRY(gemm_linear(m, s, "gemm_feature_proj", kGemmProj, w.x, M, d, cl, m->fp_w, m->fp_bias, 0, nullptr, w.h, nullptr, d));

  // positional conv: h = z + GELU(posconv(z) + bias)
  const int pad = K / 2;
  W2V2_LAUNCH(m, s, "pos_pack", launch_pos_pack(dt, w.h, B, T, rows, d, G, K, pad, w.zg, s));
  {
    GemmArgs g;
    g.role = kGemmPos;
    g.A = w.zg;
    g.lda = Cg;
    g.a_seg = (int64_t)(T + K) * Cg;
    g.seg_rows = T;
    g.a_rows = pk ? pk->pos_rows : nullptr;
    g.a_group = (int64_t)B * (T + K) * Cg;
    g.B = m->pos_w;
    g.b_group = (int64_t)Cg * K * Cg;
    g.M = M;
    g.N = Cg;
    g.K = K * Cg;
    g.groups = G;
    g.bias = m->pos_bias;
    g.bias_group = Cg;
    g.act = m->act;
    g.residual = w.h;
    g.out_f32 = w.h;
    g.ldc = d;
    g.c_group = Cg;
    W2V2_LAUNCH(m, s, "pos_conv_gemm", launch_gemm(dt, g, s));
  }
  // Post-norm: every LayerNorm writes only the GEMM operand x and the row
  // statistics; the raw residual sum stays in h, and the next residual GEMM
  // (out-proj, FFN2) applies that LayerNorm to h as it reads it.
  // Stable pre-norm: the LayerNorms feed x only and h is the plain sum.
  // fp8 mode: the operands of the four projections of every block (x for
  // qkv and fc1, the attention output, the FFN hidden) are written as e4m3
  // with their input's static scale, and those GEMMs run on e4m3 operands;
  // the CTC head keeps fp16 operands.  Calibration (m->calib): the producers
  // of those operands raise their input's amax slot instead.
  const bool stable = c.stable_layer_norm != 0;
  const bool f8 = m->fp8;
  auto slot = [&](int l, int k) { return m->calib ? m->calib + 4 * l + k : nullptr; };
  // LayerNorm of h into x for projection k (0 qkv, 2 fc1) of layer l; l equal
  // to the layer count means the CTC head
  auto ln_to_x = [&](const float* g, const float* b, float2* stats, int l, int k) {
    const bool proj = l < c.layers;
    uint8_t* y8 = (f8 && proj) ? (uint8_t*)w.x : nullptr;
    return launch_layernorm(dt, w.h, nullptr, M, d, g, b, eps, nullptr, y8 ? nullptr : w.x, 0, stats, s, y8,
                            y8 ? m->layers[l].inv[k] : 1.f, proj ? slot(l, k) : nullptr);
  };
  ResNorm rn{w.lnst, m->enc_g, m->enc_b};
  if (!stable) W2V2_LAUNCH(m, s, "layernorm", ln_to_x(m->enc_g, m->enc_b, w.lnst, 0, 0));

  for (int l = 0; l < c.layers; ++l) {
    const w2v2_model::Layer& L = m->layers[l];
    auto io = [&](int k) {
      ProjIO r;
      r.f8 = f8;
      r.col_scale = f8 ? L.cs[k] : nullptr;
      return r;
    };
    if (stable) W2V2_LAUNCH(m, s, "layernorm", ln_to_x(L.ln1_g, L.ln1_b, nullptr, l, 0));
    W2V2_TRY(gemm_linear(m, s, "gemm_qkv", kGemmQKV, w.x, M, 3 * d, d, L.wqkv, L.bqkv, 0, nullptr, nullptr, w.qkv,
                         3 * d, nullptr, io(0)));
    W2V2_LAUNCH(m, s, "attention",
                launch_attention(dt, w.qkv, w.attn, B, T, rows, c.heads, d / c.heads, w.shared, s,
                                 f8 ? (uint8_t*)w.attn : nullptr, L.inv[1], slot(l, 1)));
    W2V2_TRY(gemm_linear(m, s, "gemm_out_proj", kGemmOut, w.attn, M, d, d, L.wo, L.bo, 0, w.h, w.h, nullptr, d,
                         stable ? nullptr : &rn, io(1)));
    if (stable) {
      W2V2_LAUNCH(m, s, "layernorm", ln_to_x(L.ln2_g, L.ln2_b, nullptr, l, 2));
    } else {
      W2V2_LAUNCH(m, s, "layernorm", ln_to_x(L.ln1_g, L.ln1_b, w.lnst, l, 2));
      rn = ResNorm{w.lnst, L.ln1_g, L.ln1_b};
    }
    ProjIO io1 = io(2);
    if (f8) {
      io1.out8 = (uint8_t*)w.ffn;
      io1.out8_inv = L.inv[3];
    }
    io1.out_amax = slot(l, 3);
    W2V2_TRY(gemm_linear(m, s, "gemm_ffn1", kGemmFFN1, w.x, M, F, d, L.w1, L.b1, m->act, nullptr, nullptr, w.ffn, F,
                         nullptr, io1));
    W2V2_TRY(gemm_linear(m, s, "gemm_ffn2", kGemmFFN2, w.ffn, M, d, F, L.w2, L.b2, 0, w.h, w.h, nullptr, d,
                         stable ? nullptr : &rn, io(3)));
    if (!stable) {
      W2V2_LAUNCH(m, s, "layernorm", ln_to_x(L.ln2_g, L.ln2_b, w.lnst, l + 1, 0));
      rn = ResNorm{w.lnst, L.ln2_g, L.ln2_b};
    }
  }
  if (stable) W2V2_LAUNCH(m, s, "layernorm", ln_to_x(m->enc_g, m->enc_b, nullptr, c.layers, 0));
  if (!pk) {
    GemmArgs g;
    g.role = kGemmHead;
    g.A = w.x;
    g.lda = d;
    g.seg_rows = M;
    g.B = m->head_w;
    g.M = M;
    g.N = c.vocab;
    g.K = d;
    g.bias = m->head_b;
    g.out_f32 = logits;
    g.ldc = c.vocab;
    g.amax = keys;
    W2V2_LAUNCH(m, s, "gemm_ctc_head", launch_gemm(dt, g, s));
    return W2V2_OK;
  }
  // packed rows -> [B, T, V] through the output row table; frames past a
  // row's own frames are zero
  GemmArgs g;
  g.role = kGemmHead;
  g.A = w.x;
  g.lda = d;
  g.seg_rows = M > 0 ? M : 1;
  g.B = m->head_w;
  g.M = M;
  g.N = c.vocab;
  g.K = d;
  g.bias = m->head_b;
  g.out_f32 = logits;
  g.ldc = c.vocab;
  g.c_rows = pk->head_rows;
  g.amax = keys;
  W2V2_LAUNCH(m, s, "gemm_ctc_head", launch_gemm(dt, g, s));
  W2V2_LAUNCH(m, s, "zero_tail_frames", launch_zero_tail_frames(logits, B, T, c.vocab, rows.len, s));
  return W2V2_OK;
}

w2v2_status check_forward_args(w2v2_model* m, const void* a, const void* b, int32_t batch, const void* c) {
  if (!m) return fail(W2V2_E_ARG, "model is NULL");
  if (!a || !b || !c) return fail(W2V2_E_ARG, "a required device pointer is NULL");
  if (batch < 1 || batch > m->cfg.max_batch)
    return fail(W2V2_E_ARG, "batch must be in [1, max_batch=" + std::to_string(m->cfg.max_batch) + "]");
  return W2V2_OK;
}

// Rows [b0, b0 + n) of every workspace region, as a workspace of its own.
// base: the whole-batch regions (the model's workspace, or the static
// scratch laid out for one call's batch).
Ws ws_rows(const w2v2_model* m, const Ws& base, int b0) {
  auto at = [&](void* p, int i) { return (void*)((uint8_t*)p + (size_t)b0 * m->row_bytes[i]); };
  Ws r;
  r.bufA = at(base.bufA, 0);
  r.bufB = at(base.bufB, 1);
  r.gn_part = (double*)at(base.gn_part, 2);
  r.gn_ss = (float2*)at(base.gn_ss, 3);
  r.h = (float*)at(base.h, 4);
  r.x = at(base.x, 5);
  r.qkv = at(base.qkv, 6);
  r.attn = at(base.attn, 7);
  r.ffn = at(base.ffn, 8);
  r.zg = at(base.zg, 9);
  r.lnst = (float2*)at(base.lnst, 10);
  r.keys = (uint64_t*)at(base.keys, 11);
  return r;
}
Ws ws_rows(const w2v2_model* m, int b0) { return ws_rows(m, m->w, b0); }

// The workspace regions of a `batch`-row call packed one after another from
// `base` (256-byte aligned); *bytes receives their total size.
Ws ws_packed(const w2v2_model* m, uint8_t* base, int batch, size_t* bytes) {
  size_t off = 0;
  void* p[kWsRegions];
  for (int i = 0; i < kWsRegions; ++i) {
    p[i] = base + off;
    off += ((size_t)batch * m->row_bytes[i] + 255) & ~(size_t)255;
  }
  *bytes = off;
  Ws r;
  r.bufA = p[0];
  r.bufB = p[1];
  r.gn_part = (double*)p[2];
  r.gn_ss = (float2*)p[3];
  r.h = (float*)p[4];
  r.x = p[5];
  r.qkv = p[6];
  r.attn = p[7];
  r.ffn = p[8];
  r.zg = p[9];
  r.lnst = (float2*)p[10];
  r.keys = (uint64_t*)p[11];
  return r;
}

// Whole network on rows [b0, b0 + n) of the batch, on stream s.
// decode: the head also raises the rows' argmax keys (w.keys).
w2v2_status forward_rows(w2v2_model* m, const Ws& base, const float* pcm, const int32_t* valid, int b0, int n,
                         float* logits, hipStream_t s, bool shared = false, bool decode = false) {
  Ws w = ws_rows(m, base, b0);
  w.shared = shared;
  const void* feat = nullptr;
  // profiling "stage": one event pair around this part's frontend and one
  // around its encoder + head, on the part's own stream
  const bool stage = m->prof_on && m->prof_only == "stage";
  if (stage) m->prof->before("stage_frontend", s);
  W2V2_TRY(run_frontend(m, w, pcm + (size_t)b0 * m->cfg.window, valid + b0, n, s, &feat));
  if (stage) {
    m->prof->after("stage_frontend", s);
    m->prof->before("stage_encoder", s);
  }
  W2V2_TRY(run_encoder(m, w, feat, n, logits + (size_t)b0 * m->Tf * m->cfg.vocab, s, nullptr,
                       decode ? w.keys : nullptr));
  if (stage) m->prof->after("stage_encoder", s);
  return W2V2_OK;
}

// One row range [b0, b0 + nb) of a true-length call on stream s: its packing
// (device spans and starts relative to the range's own packed rows, already
// uploaded), its row tables in the range's share of each table region, then
// the frontend and encoder on the range's workspace slice.
w2v2_status true_length_rows(w2v2_model* m, const float* pcm, int b0, int nb, const int64_t* P, float* logits,
                             hipStream_t s, bool shared = false) {
  const w2v2_config& c = m->cfg;
  const int n = c.n_conv, Bm = c.max_batch;
  const int32_t* dlen = m->tl_i32;
  const int32_t* dstart = m->tl_i32 + (size_t)n * Bm;
  const int32_t* dvalid = m->tl_i32 + (size_t)2 * n * Bm;
  Packing pk;
  for (int i = 0; i < n; ++i) {
    pk.P[i] = P[i];
    pk.lvl[i].len = dlen + (size_t)i * Bm + b0;
    pk.lvl[i].start = dstart + (size_t)i * Bm + b0;
  }
  const int Tf = m->Tf, Cg = c.hidden / c.pos_groups;
  RowTable tabs[kMaxRowTables];
  int nt = 0, tmax = 1;
  int64_t off = 0;  // each table region holds Bm * frames entries; this range uses rows b0 .. b0 + nb of it
  for (int i = 1; i < n; ++i) {
    tabs[nt] = RowTable{pk.lvl[i].start, pk.lvl[i].len, m->tl_base + (size_t)(i - 1) * Bm + b0,
                        (int64_t)c.conv_stride[i] * c.conv_dim[i - 1], m->tl_rows + off + (int64_t)b0 * m->T[i]};
    pk.a_rows[i] = tabs[nt].out;
    off += (int64_t)Bm * m->T[i];
    tmax = std::max(tmax, m->T[i]);
    ++nt;
  }
  tabs[nt] = RowTable{pk.lvl[n - 1].start, pk.lvl[n - 1].len, m->tl_base + (size_t)(n - 1) * Bm + b0, Cg,
                      m->tl_rows + off + (int64_t)b0 * Tf};
  pk.pos_rows = tabs[nt++].out;
  off += (int64_t)Bm * Tf;
  tabs[nt] = RowTable{pk.lvl[n - 1].start, pk.lvl[n - 1].len, m->tl_base + (size_t)n * Bm + b0, c.vocab,
                      m->tl_rows + off + (int64_t)b0 * Tf};
  pk.head_rows = tabs[nt++].out;
  tmax = std::max(tmax, Tf);
  W2V2_LAUNCH(m, s, "row_tables", launch_row_tables(tabs, nt, nb, tmax, s));

  Ws w = ws_rows(m, b0);
  w.shared = shared;
  const void* feat = nullptr;
  W2V2_TRY(run_frontend(m, w, pcm + (size_t)b0 * c.window, dvalid + b0, nb, s, &feat, &pk));
  return run_encoder(m, w, feat, nb, logits + (size_t)b0 * Tf * c.vocab, s, &pk);
}

// w2v2_forward, and with ids / lens set w2v2_forward_greedy: the head then
// raises each frame's argmax key and the keys are collapsed into ids.
// ws: the whole-batch workspace regions (null: the model's).
w2v2_status forward_impl(w2v2_model* m, const float* pcm, const int32_t* valid, int32_t batch, float* logits,
                         int32_t* vframes, int32_t* ids, int32_t* lens, void* stream, const Ws* ws = nullptr) {
  W2V2_TRY(check_forward_args(m, pcm, valid, batch, logits));
  DeviceGuard guard(m->device);
  hipStream_t s = (hipStream_t)stream;
  const Ws& base = ws ? *ws : m->w;
  const bool decode = ids != nullptr;
  if (decode) W2V2_LAUNCH(m, s, "zero_keys", launch_zero_keys(base.keys, (int64_t)batch * m->Tf, s));
  // profiling every kernel (no filter) runs the batch as one pass, so that each
  // kernel's event-timed duration is its own and not shared with the other half
  const bool serial = batch == 1 || (m->prof_on && m->prof_only.empty());
  if (serial) {
    W2V2_TRY(forward_rows(m, base, pcm, valid, 0, batch, logits, s, false, decode));
  } else {
    // The batch is cut into np near-equal row ranges that run concurrently,
    // the first on the caller's stream and the others on the model's own
    // streams, so that one part's latency-bound kernels (attention, norms,
    // GEMM tails) overlap the other parts' work.  Rows are independent: the
    // results are the bits of a single-stream run.
    const int np = std::min(batch, kSplit);
    if (hipEventRecord(m->ev_fork, s) != hipSuccess) return fail(W2V2_E_DEVICE, "fork of the streams failed");
    for (int p = 1; p < np; ++p)
      if (hipStreamWaitEvent(m->aux[p], m->ev_fork, 0) != hipSuccess)
        return fail(W2V2_E_DEVICE, "fork of the streams failed");
    w2v2_status st = W2V2_OK;
    int b0 = 0;
    for (int p = 0; p < np && st == W2V2_OK; ++p) {
      const int n = batch / np + (p < batch % np ? 1 : 0);
      st = forward_rows(m, base, pcm, valid, b0, n, logits, p == 0 ? s : m->aux[p], np > 1, decode);
      b0 += n;
    }
    // the caller's stream waits for every part whatever happened
    for (int p = 1; p < np; ++p)
      if (hipEventRecord(m->ev_join[p], m->aux[p]) != hipSuccess || hipStreamWaitEvent(s, m->ev_join[p], 0) != hipSuccess)
        return fail(W2V2_E_DEVICE, "join of the streams failed");
    if (st != W2V2_OK) return st;
  }
  if (vframes)
    W2V2_LAUNCH(m, s, "valid_frames",
                launch_valid_frames(valid, batch, m->cfg.window, m->cfg.n_conv, m->cfg.conv_kernel,
                                    m->cfg.conv_stride, vframes, s));
  if (decode)
    W2V2_LAUNCH(m, s, "ctc_collapse",
                launch_ctc_collapse_keys(base.keys, vframes, batch, m->Tf, m->cfg.blank_id, ids, lens, s));
  return W2V2_OK;
}

}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------
extern "C" {

const char* w2v2_last_error(void) { return g_last_error.c_str(); }

w2v2_status w2v2_create(const w2v2_config* cfgp, const w2v2_tensor* weights, int32_t n_weights, int32_t device,
                        w2v2_model** out) {
  g_last_error.clear();
  if (!out) return fail(W2V2_E_ARG, "out is NULL");
  *out = nullptr;
  if (!cfgp) return fail(W2V2_E_ARG, "cfg is NULL");
  if (n_weights < 0) return fail(W2V2_E_ARG, "n_weights < 0");
  const w2v2_config c = *cfgp;
  int frames = 0;
  const std::string cerr = check_config(c, &frames);
  if (!cerr.empty()) return fail(W2V2_E_CONFIG, cerr);

  // ---- weight table ----
  if (n_weights == 0 || !weights) return fail(W2V2_E_WEIGHTS, "weight table is empty");
  const std::vector<ExpectedW> exp = expected_weights(c);
  std::map<std::string, const w2v2_tensor*> got;
  for (int i = 0; i < n_weights; ++i) {
    const w2v2_tensor& t = weights[i];
    if (!t.name) return fail(W2V2_E_WEIGHTS, "weight " + std::to_string(i) + " has no name");
    if (got.count(t.name)) return fail(W2V2_E_WEIGHTS, std::string("duplicate weight ") + t.name);
    got[t.name] = &t;
  }
  for (const auto& e : exp) {
    auto it = got.find(e.name);
    if (it == got.end()) return fail(W2V2_E_WEIGHTS, "missing weight " + e.name);
    const w2v2_tensor& t = *it->second;
    if (!t.data) return fail(W2V2_E_WEIGHTS, "weight " + e.name + " has no data");
    if (t.ndim < 1 || t.ndim > 4) return fail(W2V2_E_WEIGHTS, "weight " + e.name + " has bad ndim");
    std::vector<int64_t> sh(t.shape, t.shape + t.ndim);
    bool ok = (sh == e.shape);
    if (!ok && e.name == "pos.weight_g" && sh.size() == 3 && sh[0] == 1 && sh[1] == 1 && sh[2] == e.shape[0])
      ok = true;
    if (!ok) return fail(W2V2_E_WEIGHTS, "weight " + e.name + " has the wrong shape");
    int64_t n = 1;
    for (auto v : e.shape) n *= v;
    for (int64_t j = 0; j < n; ++j)
      if (!std::isfinite(t.data[j])) return fail(W2V2_E_WEIGHTS, "weight " + e.name + " has a non-finite value");
    static const std::string kAmax = ".input_amax";
    if (e.name.size() > kAmax.size() && e.name.compare(e.name.size() - kAmax.size(), kAmax.size(), kAmax) == 0 &&
        !(t.data[0] > 0.f))
      return fail(W2V2_E_WEIGHTS, "weight " + e.name + " must be positive");
  }
  if ((size_t)n_weights != exp.size()) {
    for (const auto& kv : got) {
      bool known = false;
      for (const auto& e : exp) known = known || (e.name == kv.first);
      if (!known) return fail(W2V2_E_WEIGHTS, "unknown weight " + kv.first);
    }
    return fail(W2V2_E_WEIGHTS, "weight table has the wrong number of entries");
  }
  auto W = [&](const std::string& n) { return got[n]->data; };
  auto Wv = [&](const std::string& n, size_t count) {
    const float* p = W(n);
    return std::vector<float>(p, p + count);
  };

  // ---- device ----
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return fail(W2V2_E_DEVICE, "no HIP device");
  if (device < 0 || device >= ndev) return fail(W2V2_E_DEVICE, "device index out of range");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return fail(W2V2_E_DEVICE, "hipGetDeviceProperties failed");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(W2V2_E_DEVICE, std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950");
  DeviceGuard guard(device);

  w2v2_model* m = new w2v2_model();
  m->cfg = c;
  m->device = device;
  m->dt = (c.precision == W2V2_FP32 || c.precision == W2V2_FP8_ON_FP32) ? DType::F32 : DType::F16;
  m->fp8 = c.precision == W2V2_FP8 || c.precision == W2V2_FP8_ON_FP32;
  m->act = c.gelu_kind == W2V2_GELU_TANH ? 2 : 1;
  {
    int64_t n = c.window;
    for (int i = 0; i < c.n_conv; ++i) {
      n = conv_len(n, c.conv_kernel[i], c.conv_stride[i]);
      m->T[i] = (int)n;
    }
    m->Tf = frames;
  }
  const DType dt = m->dt;
  const int d = c.hidden, F = c.ffn, G = c.pos_groups, Cg = d / G, K = c.pos_kernel;
  const int cl = c.conv_dim[c.n_conv - 1];

  // ---- pack weights ----
  Arena ar;
  struct Off {
    size_t w = 0, b = 0, g = 0, be = 0;
    bool hb = false, hn = false;
  };
  std::vector<Off> conv_off(c.n_conv);
  int cin = 1;
  for (int i = 0; i < c.n_conv; ++i) {
    const int co = c.conv_dim[i], k = c.conv_kernel[i];
    const std::string p = "fe.conv" + std::to_string(i);
    const float* w = W(p + ".weight");
    if (i == 0) {
      conv_off[i].w = add_f32(ar, std::vector<float>(w, w + (size_t)co * k));
    } else {
      std::vector<float> r((size_t)co * k * cin);
      for (int o = 0; o < co; ++o)
        for (int ci = 0; ci < cin; ++ci)
          for (int j = 0; j < k; ++j) r[((size_t)o * k + j) * cin + ci] = w[((size_t)o * cin + ci) * k + j];
      conv_off[i].w = add_t(ar, dt, r);
    }
    if (c.conv_bias) {
      conv_off[i].b = add_f32(ar, Wv(p + ".bias", co));
      conv_off[i].hb = true;
    }
    if (c.feat_norm == W2V2_NORM_LAYER || i == 0) {
      const std::string n = "fe.norm" + std::to_string(i);
      conv_off[i].g = add_f32(ar, Wv(n + ".weight", co));
      conv_off[i].be = add_f32(ar, Wv(n + ".bias", co));
      conv_off[i].hn = true;
    }
    cin = co;
  }
  const size_t o_fpg = add_f32(ar, Wv("fp.norm.weight", cl));
  const size_t o_fpb = add_f32(ar, Wv("fp.norm.bias", cl));
  const size_t o_fpw = add_t(ar, dt, Wv("fp.proj.weight", (size_t)d * cl));
  const size_t o_fpbias = add_f32(ar, Wv("fp.proj.bias", d));
  size_t o_posw, o_posb;
  {
    // weight norm folded per tap: w[o, i, k] = g[k] v[o, i, k] / ||v[:, :, k]||_F
    const float* v = W("pos.weight_v");
    const float* gk = W("pos.weight_g");
    std::vector<double> scale(K);
    for (int k = 0; k < K; ++k) {
      double ss = 0.0;
      for (int o = 0; o < d; ++o)
        for (int i = 0; i < Cg; ++i) {
          const double x = v[((size_t)o * Cg + i) * K + k];
          ss += x * x;
        }
      scale[k] = ss > 0.0 ? (double)gk[k] / std::sqrt(ss) : 0.0;
    }
    // [G][Cg_out][K*Cg_in], K index = k*Cg + i
    std::vector<float> r((size_t)d * K * Cg);
    for (int g = 0; g < G; ++g)
      for (int ol = 0; ol < Cg; ++ol) {
        const int o = g * Cg + ol;
        for (int k = 0; k < K; ++k)
          for (int i = 0; i < Cg; ++i)
            r[(((size_t)g * Cg + ol) * K + k) * Cg + i] = (float)(v[((size_t)o * Cg + i) * K + k] * scale[k]);
      }
    o_posw = add_t(ar, dt, r);
    o_posb = add_f32(ar, Wv("pos.bias", d));
  }
  const size_t o_encg = add_f32(ar, Wv("enc.norm.weight", d));
  const size_t o_encb = add_f32(ar, Wv("enc.norm.bias", d));
  struct LOff {
    size_t wqkv, wo, w1, w2, bqkv, bo, b1, b2, g1, be1, g2, be2;
    size_t cs[4] = {0, 0, 0, 0};
  };
  std::vector<LOff> loff(c.layers);
  for (int l = 0; l < c.layers; ++l) {
    const std::string p = "layer" + std::to_string(l) + ".";
    std::vector<float> qkv((size_t)3 * d * d), bq((size_t)3 * d);
    const char* pr[3] = {"q", "k", "v"};
    for (int j = 0; j < 3; ++j) {
      memcpy(qkv.data() + (size_t)j * d * d, W(p + "attn." + pr[j] + ".weight"), sizeof(float) * d * d);
      memcpy(bq.data() + (size_t)j * d, W(p + "attn." + pr[j] + ".bias"), sizeof(float) * d);
    }
    if (m->fp8) {
      // per-tensor weight scales of q, k and v; the activation scale of
      // their shared input
      std::vector<double> sw(3);
      for (int j = 0; j < 3; ++j) sw[j] = amax_of(qkv.data() + (size_t)j * d * d, (size_t)d * d) / 448.0;
      loff[l].wqkv = add_e4m3(ar, qkv, {sw[0], sw[1], sw[2]}, (size_t)d * d);
      const double ax = W(p + "attn.qkv.input_amax")[0];
      std::vector<float> cs((size_t)3 * d);
      for (int j = 0; j < 3; ++j)
        for (int n = 0; n < d; ++n) cs[(size_t)j * d + n] = (float)(ax / 448.0 * sw[j]);
      loff[l].cs[0] = add_f32(ar, cs);
    } else {
      loff[l].wqkv = add_t(ar, dt, qkv);
    }
    loff[l].bqkv = add_f32(ar, bq);
    loff[l].wo = m->fp8 ? add_fp8_linear(ar, Wv(p + "attn.out.weight", (size_t)d * d), W(p + "attn.out.input_amax")[0],
                                         d, &loff[l].cs[1])
                        : add_t(ar, dt, Wv(p + "attn.out.weight", (size_t)d * d));
    loff[l].bo = add_f32(ar, Wv(p + "attn.out.bias", d));
    loff[l].g1 = add_f32(ar, Wv(p + "attn_norm.weight", d));
    loff[l].be1 = add_f32(ar, Wv(p + "attn_norm.bias", d));
    loff[l].w1 = m->fp8 ? add_fp8_linear(ar, Wv(p + "ffn.fc1.weight", (size_t)F * d), W(p + "ffn.fc1.input_amax")[0],
                                         F, &loff[l].cs[2])
                        : add_t(ar, dt, Wv(p + "ffn.fc1.weight", (size_t)F * d));
    loff[l].b1 = add_f32(ar, Wv(p + "ffn.fc1.bias", F));
    loff[l].w2 = m->fp8 ? add_fp8_linear(ar, Wv(p + "ffn.fc2.weight", (size_t)d * F), W(p + "ffn.fc2.input_amax")[0],
                                         d, &loff[l].cs[3])
                        : add_t(ar, dt, Wv(p + "ffn.fc2.weight", (size_t)d * F));
    loff[l].b2 = add_f32(ar, Wv(p + "ffn.fc2.bias", d));
    loff[l].g2 = add_f32(ar, Wv(p + "ffn_norm.weight", d));
    loff[l].be2 = add_f32(ar, Wv(p + "ffn_norm.bias", d));
  }
  const size_t o_hw = add_t(ar, dt, Wv("head.weight", (size_t)c.vocab * d));
  const size_t o_hb = add_f32(ar, Wv("head.bias", c.vocab));

  m->wbytes = ar.bytes.size();
  if (hipMalloc(&m->wmem, m->wbytes) != hipSuccess) {
    (void)hipGetLastError();
    delete m;
    return fail(W2V2_E_NOMEM, "cannot allocate " + std::to_string(ar.bytes.size()) + " bytes of weights");
  }
  if (hipMemcpy(m->wmem, ar.bytes.data(), m->wbytes, hipMemcpyHostToDevice) != hipSuccess) {
    delete m;
    return fail(W2V2_E_DEVICE, "weight upload failed");
  }
  auto P = [&](size_t off) { return (const void*)((const uint8_t*)m->wmem + off); };
  auto PF = [&](size_t off) { return (const float*)P(off); };
  for (int i = 0; i < c.n_conv; ++i) {
    m->conv[i].w = P(conv_off[i].w);
    m->conv[i].bias = conv_off[i].hb ? PF(conv_off[i].b) : nullptr;
    m->conv[i].gamma = conv_off[i].hn ? PF(conv_off[i].g) : nullptr;
    m->conv[i].beta = conv_off[i].hn ? PF(conv_off[i].be) : nullptr;
  }
  m->fp_g = PF(o_fpg);
  m->fp_b = PF(o_fpb);
  m->fp_w = P(o_fpw);
  m->fp_bias = PF(o_fpbias);
  m->pos_w = P(o_posw);
  m->pos_bias = PF(o_posb);
  m->enc_g = PF(o_encg);
  m->enc_b = PF(o_encb);
  m->layers.resize(c.layers);
  for (int l = 0; l < c.layers; ++l) {
    auto& L = m->layers[l];
    L.wqkv = P(loff[l].wqkv);
    L.bqkv = PF(loff[l].bqkv);
    L.wo = P(loff[l].wo);
    L.bo = PF(loff[l].bo);
    L.w1 = P(loff[l].w1);
    L.b1 = PF(loff[l].b1);
    L.w2 = P(loff[l].w2);
    L.b2 = PF(loff[l].b2);
    L.ln1_g = PF(loff[l].g1);
    L.ln1_b = PF(loff[l].be1);
    L.ln2_g = PF(loff[l].g2);
    L.ln2_b = PF(loff[l].be2);
    if (m->fp8) {
      const std::string p = "layer" + std::to_string(l) + ".";
      for (int k = 0; k < 4; ++k) {
        L.cs[k] = PF(loff[l].cs[k]);
        L.inv[k] = (float)(448.0 / (double)W(p + kFp8Inputs[k] + ".input_amax")[0]);
      }
    }
  }
  m->head_w = P(o_hw);
  m->head_b = PF(o_hb);

  // ---- workspace ----
  const int64_t Bm = c.max_batch;
  const size_t ds = dsize(dt);
  int64_t elA = 0, elB = 0;
  for (int i = 0; i < c.n_conv; ++i) {
    const int64_t e = Bm * m->T[i] * c.conv_dim[i];
    if (i & 1) elB = std::max(elB, e);
    else elA = std::max(elA, e);
  }
  const int64_t M = Bm * m->Tf;
  elA = std::max(elA, M * cl);  // w2v2_forward_encoder stages its input features here
  std::vector<size_t> sizes = {
      (size_t)elA * ds,                                   // bufA
      (size_t)std::max<int64_t>(elB, 1) * ds,             // bufB
      (size_t)(Bm * gn0_partial_doubles(c.conv_kernel[0], m->T[0]) * 8),  // gn_part
      (size_t)Bm * c.conv_dim[0] * 8,                     // gn_ss
      (size_t)M * d * 4,                                  // h
      (size_t)M * std::max(d, cl) * ds,                   // x
      (size_t)M * 3 * d * ds,                             // qkv
      (size_t)M * d * ds,                                 // attn
      (size_t)M * F * ds,                                 // ffn
      (size_t)G * Bm * (m->Tf + K) * Cg * ds,             // zg
      (size_t)M * 8,                                      // lnst
      (size_t)M * 8,                                      // keys
      (size_t)tl_i32_words(c) * 4 + (size_t)(c.n_conv + 1) * Bm * 8,   // true-length lengths/starts + bases
      (size_t)tl_rows_count(c, m->T, m->Tf) * 8,          // true-length row tables
  };
  size_t total = 0;
  std::vector<size_t> offs;
  for (size_t sz : sizes) {
    offs.push_back(total);
    total += (sz + 255) & ~size_t(255);
  }
  m->wsbytes = total;
  if (hipMalloc(&m->ws, total) != hipSuccess) {
    (void)hipGetLastError();
    delete m;
    return fail(W2V2_E_NOMEM, "cannot allocate " + std::to_string(total) + " bytes of workspace");
  }
  uint8_t* wsb = (uint8_t*)m->ws;
  m->w.bufA = wsb + offs[0];
  m->w.bufB = wsb + offs[1];
  m->w.gn_part = (double*)(wsb + offs[2]);
  m->w.gn_ss = (float2*)(wsb + offs[3]);
  m->w.h = (float*)(wsb + offs[4]);
  m->w.x = wsb + offs[5];
  m->w.qkv = wsb + offs[6];
  m->w.attn = wsb + offs[7];
  m->w.ffn = wsb + offs[8];
  m->w.zg = wsb + offs[9];
  m->w.lnst = (float2*)(wsb + offs[10]);
  m->w.keys = (uint64_t*)(wsb + offs[11]);
  for (int i = 0; i < kWsRegions; ++i) m->row_bytes[i] = sizes[i] / (size_t)Bm;
  if (hipEventCreateWithFlags(&m->ev_fork, hipEventDisableTiming) != hipSuccess) {
    m->ev_fork = nullptr;
    delete m;
    return fail(W2V2_E_DEVICE, "hipEventCreate failed");
  }
  for (int i = 1; i < kSplit; ++i) {
    if (hipStreamCreateWithFlags(&m->aux[i], hipStreamNonBlocking) != hipSuccess) {
      m->aux[i] = nullptr;
      delete m;
      return fail(W2V2_E_DEVICE, "hipStreamCreate failed");
    }
    if (hipEventCreateWithFlags(&m->ev_join[i], hipEventDisableTiming) != hipSuccess) {
      m->ev_join[i] = nullptr;
      delete m;
      return fail(W2V2_E_DEVICE, "hipEventCreate failed");
    }
  }
  m->tl_i32 = (int32_t*)(wsb + offs[12]);
  m->tl_base = (int64_t*)(wsb + offs[12] + (size_t)tl_i32_words(c) * 4);
  m->tl_rows = (int64_t*)(wsb + offs[13]);
  // pinned staging of the true-length tables (lengths, starts, valid, bases)
  m->tl_bytes = (size_t)tl_i32_words(c) * 4 + (size_t)(c.n_conv + 1) * Bm * 8;
  if (hipHostMalloc((void**)&m->tl_pinned, m->tl_bytes, hipHostMallocDefault) != hipSuccess) {
    m->tl_pinned = nullptr;
    (void)hipGetLastError();
    delete m;
    return fail(W2V2_E_NOMEM, "cannot allocate pinned staging for the row lengths");
  }
  if (hipEventCreateWithFlags(&m->tl_copied, hipEventDisableTiming) != hipSuccess) {
    m->tl_copied = nullptr;
    delete m;
    return fail(W2V2_E_DEVICE, "hipEventCreate failed");
  }
  // the device address of this device's static scratch
  if (scratch_setup(device, &m->scratch) != hipSuccess) {
    (void)hipGetLastError();
    delete m;
    return fail(W2V2_E_DEVICE, "cannot resolve the device address of the static scratch");
  }
  if (hipDeviceSynchronize() != hipSuccess) {
    delete m;
    return fail(W2V2_E_DEVICE, "device synchronization failed after weight upload");
  }
  *out = m;
  return W2V2_OK;
}

void w2v2_destroy(w2v2_model* m) {
  if (!m) return;
  DeviceGuard guard(m->device);
  delete m;
}

w2v2_status w2v2_num_frames(const w2v2_model* m, int64_t samples, int32_t* frames) {
  if (!m || !frames) return fail(W2V2_E_ARG, "NULL argument");
  if (samples < 0) return fail(W2V2_E_ARG, "samples < 0");
  int64_t n = samples;
  for (int i = 0; i < m->cfg.n_conv; ++i) n = conv_len(n, m->cfg.conv_kernel[i], m->cfg.conv_stride[i]);
  *frames = (int32_t)n;
  return W2V2_OK;
}

w2v2_status w2v2_model_info(const w2v2_model* m, int32_t* frames_per_window, int32_t* vocab,
                            int64_t* workspace_bytes) {
  if (!m) return fail(W2V2_E_ARG, "model is NULL");
  if (frames_per_window) *frames_per_window = m->Tf;
  if (vocab) *vocab = m->cfg.vocab;
  if (workspace_bytes) *workspace_bytes = (int64_t)m->wsbytes;
  return W2V2_OK;
}

w2v2_status w2v2_forward(w2v2_model* m, const float* pcm, const int32_t* valid, int32_t batch, float* logits,
                         int32_t* vframes, void* stream) {
  return forward_impl(m, pcm, valid, batch, logits, vframes, nullptr, nullptr, stream);
}

w2v2_status w2v2_forward_greedy(w2v2_model* m, const float* pcm, const int32_t* valid, int32_t batch,
                                float* logits, int32_t* vframes, int32_t* ids, int32_t* lens, void* stream) {
  if (!vframes || !ids || !lens) return fail(W2V2_E_ARG, "vframes, ids and lens must not be NULL");
  return forward_impl(m, pcm, valid, batch, logits, vframes, ids, lens, stream);
}

w2v2_status w2v2_forward_greedy_noalloc(w2v2_model* m, const float* pcm, const int32_t* valid, int32_t batch,
                                        float* logits, int32_t* vframes, int32_t* ids, int32_t* lens,
                                        void* stream) {
  W2V2_TRY(check_forward_args(m, pcm, valid, batch, logits));
  if (!vframes || !ids || !lens) return fail(W2V2_E_ARG, "vframes, ids and lens must not be NULL");
  if (!m->scratch) return fail(W2V2_E_DEVICE, "the static scratch has no device address");
  size_t need = 0;
  const Ws ws = ws_packed(m, (uint8_t*)m->scratch, batch, &need);
  if (need > kScratchBytes)
    return fail(W2V2_E_ARG, "batch " + std::to_string(batch) + " needs " + std::to_string(need) +
                                " bytes of scratch; w2v2_forward_greedy_noalloc holds " +
                                std::to_string(kScratchBytes));
  return forward_impl(m, pcm, valid, batch, logits, vframes, ids, lens, stream, &ws);
}

w2v2_status w2v2_calibrate(w2v2_model* m, const float* pcm, const int32_t* valid, int32_t batch, float* logits,
                           float* amax, void* stream) {
  if (!m) return fail(W2V2_E_ARG, "model is NULL");
  if (!amax) return fail(W2V2_E_ARG, "amax is NULL");
  if (m->fp8) return fail(W2V2_E_ARG, "calibrate with an fp32 or fp16 model, not an fp8 one");
  m->calib = amax;
  const w2v2_status st = forward_impl(m, pcm, valid, batch, logits, nullptr, nullptr, nullptr, stream);
  m->calib = nullptr;
  return st;
}

w2v2_status w2v2_forward_true_length(w2v2_model* m, const float* pcm, const int32_t* valid_host, int32_t batch,
                                     float* logits, int32_t* vframes, void* stream) {
  W2V2_TRY(check_forward_args(m, pcm, valid_host, batch, logits));
  const w2v2_config& c = m->cfg;
  const int n = c.n_conv, B = batch, Bm = c.max_batch;
  for (int b = 0; b < B; ++b)
    if (valid_host[b] < 0 || valid_host[b] > c.window)
      return fail(W2V2_E_ARG, "valid[" + std::to_string(b) + "] must be in [0, window]");
  DeviceGuard guard(m->device);
  hipStream_t s = (hipStream_t)stream;

  // Like w2v2_forward, the rows are cut into near-equal ranges that run
  // concurrently (profiling every kernel: one range).  Each range is packed
  // on its own: its rows' frames are consecutive from the start of its
  // workspace slice.
  const bool serial = B == 1 || (m->prof_on && m->prof_only.empty());
  const int np = serial ? 1 : std::min(B, kSplit);
  int r0[kSplit + 1] = {};
  for (int p = 0; p < np; ++p) r0[p + 1] = r0[p] + B / np + (p < B % np ? 1 : 0);

  // host: frames and packed starts of every row at every conv level, staged
  // in pinned memory; the previous call's upload from it must have finished
  const int64_t words = tl_i32_words(c);
  if (m->tl_pending && hipEventSynchronize(m->tl_copied) != hipSuccess)
    return fail(W2V2_E_DEVICE, "waiting for the previous upload failed");
  m->tl_pending = false;
  int64_t* blob = m->tl_pinned;
  std::memset(blob, 0, m->tl_bytes);
  int32_t* len = (int32_t*)blob;                     // [n][Bm]
  int32_t* start = len + (size_t)n * Bm;             // [n][Bm], relative to the row's range
  int32_t* vcopy = start + (size_t)n * Bm;           // [Bm]
  int64_t* base = blob + words / 2;                  // [n + 1][Bm]
  int64_t P[kSplit][W2V2_MAX_CONV] = {};
  for (int b = 0; b < B; ++b) {
    vcopy[b] = valid_host[b];
    int64_t f = valid_host[b];
    for (int i = 0; i < n; ++i) {
      f = conv_len(f, c.conv_kernel[i], c.conv_stride[i]);
      len[(size_t)i * Bm + b] = (int32_t)f;
    }
  }
  for (int p = 0; p < np; ++p)
    for (int i = 0; i < n; ++i) {
      int64_t acc = 0;
      for (int b = r0[p]; b < r0[p + 1]; ++b) {
        start[(size_t)i * Bm + b] = (int32_t)acc;
        acc += len[(size_t)i * Bm + b];
      }
      P[p][i] = acc;
    }
  // table bases: conv i reads row b's input window at packed input row
  // start_{i-1}[b] + t * stride_i; the positional conv reads row b's padded
  // segment of T + K frames; the head writes row b's frame t at (b * T + t) * V
  // (row b counted from the first row of its range)
  const int Tf = m->Tf, K = c.pos_kernel, Cg = c.hidden / c.pos_groups;
  for (int p = 0; p < np; ++p)
    for (int b = r0[p]; b < r0[p + 1]; ++b) {
      for (int i = 1; i < n; ++i)
        base[(size_t)(i - 1) * Bm + b] = (int64_t)start[(size_t)(i - 1) * Bm + b] * c.conv_dim[i - 1];
      base[(size_t)(n - 1) * Bm + b] = (int64_t)(b - r0[p]) * (Tf + K) * Cg;
      base[(size_t)n * Bm + b] = (int64_t)(b - r0[p]) * Tf * c.vocab;
    }
  if (hipMemcpyAsync(m->tl_i32, blob, m->tl_bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
      hipEventRecord(m->tl_copied, s) != hipSuccess)
    return fail(W2V2_E_DEVICE, "upload of the row lengths failed");
  m->tl_pending = true;

  if (np == 1) {
    W2V2_TRY(true_length_rows(m, pcm, 0, B, P[0], logits, s));
  } else {
    // the fork follows the upload, so every range sees the tables
    if (hipEventRecord(m->ev_fork, s) != hipSuccess) return fail(W2V2_E_DEVICE, "fork of the streams failed");
    for (int p = 1; p < np; ++p)
      if (hipStreamWaitEvent(m->aux[p], m->ev_fork, 0) != hipSuccess)
        return fail(W2V2_E_DEVICE, "fork of the streams failed");
    w2v2_status st = W2V2_OK;
    for (int p = 0; p < np && st == W2V2_OK; ++p)
      st = true_length_rows(m, pcm, r0[p], r0[p + 1] - r0[p], P[p], logits, p == 0 ? s : m->aux[p], true);
    for (int p = 1; p < np; ++p)
      if (hipEventRecord(m->ev_join[p], m->aux[p]) != hipSuccess || hipStreamWaitEvent(s, m->ev_join[p], 0) != hipSuccess)
        return fail(W2V2_E_DEVICE, "join of the streams failed");
    if (st != W2V2_OK) return st;
  }
  if (vframes)
    W2V2_LAUNCH(m, s, "valid_frames",
                launch_valid_frames(m->tl_i32 + (size_t)2 * n * Bm, B, c.window, c.n_conv, c.conv_kernel,
                                    c.conv_stride, vframes, s));
  return W2V2_OK;
}

w2v2_status w2v2_forward_frontend(w2v2_model* m, const float* pcm, const int32_t* valid, int32_t batch,
                                  float* features, void* stream) {
  W2V2_TRY(check_forward_args(m, pcm, valid, batch, features));
  DeviceGuard guard(m->device);
  hipStream_t s = (hipStream_t)stream;
  const void* feat = nullptr;
  W2V2_TRY(run_frontend(m, m->w, pcm, valid, batch, s, &feat));
  const int64_t n = (int64_t)batch * m->Tf * m->cfg.conv_dim[m->cfg.n_conv - 1];
  W2V2_LAUNCH(m, s, "cast_to_f32", launch_cast_to_f32(m->dt, feat, features, n, s));
  return W2V2_OK;
}

w2v2_status w2v2_forward_encoder(w2v2_model* m, const float* features, int32_t batch, float* logits,
                                 void* stream) {
  W2V2_TRY(check_forward_args(m, features, features, batch, logits));
  DeviceGuard guard(m->device);
  hipStream_t s = (hipStream_t)stream;
  const int64_t n = (int64_t)batch * m->Tf * m->cfg.conv_dim[m->cfg.n_conv - 1];
  W2V2_LAUNCH(m, s, "cast_from_f32", launch_cast_from_f32(m->dt, features, m->w.bufA, n, s));
  W2V2_TRY(run_encoder(m, m->w, m->w.bufA, batch, logits, s));
  return W2V2_OK;
}

w2v2_status w2v2_ctc_greedy(const float* logits, const int32_t* vframes, int32_t batch, int32_t frames,
                            int32_t vocab, int32_t blank_id, int32_t* ids, int32_t* lens, void* stream) {
  if (!logits || !vframes || !ids || !lens) return fail(W2V2_E_ARG, "a required device pointer is NULL");
  if (batch < 1) return fail(W2V2_E_ARG, "batch must be >= 1");
  if (frames < 1 || frames > 16384) return fail(W2V2_E_ARG, "frames must be in [1, 16384]");
  if (vocab < 1) return fail(W2V2_E_ARG, "vocab must be >= 1");
  if (blank_id < 0 || blank_id >= vocab) return fail(W2V2_E_ARG, "blank_id must be in [0, vocab)");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_frame_argmax(logits, (int64_t)batch * frames, vocab, ids, s);
  if (e == hipSuccess) e = launch_ctc_collapse(vframes, batch, frames, blank_id, ids, lens, s);
  if (e != hipSuccess) return fail(W2V2_E_DEVICE, std::string("ctc_greedy: ") + hipGetErrorString(e));
  return W2V2_OK;
}

w2v2_status w2v2_profile_enable(w2v2_model* m, int32_t enable, const char* only) {
  if (!m) return fail(W2V2_E_ARG, "model is NULL");
  if (enable && !m->prof) m->prof = new Profiler();
  m->prof_on = enable != 0;
  m->prof_only = only ? only : "";
  return W2V2_OK;
}

w2v2_status w2v2_profile_read(w2v2_model* m, int32_t cap, const char** names, double* total_ms,
                              int64_t* launches, int32_t* n) {
  if (!m || !n || cap < 0 || (cap > 0 && (!names || !total_ms || !launches)))
    return fail(W2V2_E_ARG, "bad argument");
  *n = 0;
  if (!m->prof) return W2V2_OK;
  DeviceGuard guard(m->device);
  Profiler& p = *m->prof;
  if (p.err != hipSuccess) return fail(W2V2_E_DEVICE, std::string("profiling: ") + hipGetErrorString(p.err));
  for (auto& r : p.recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(W2V2_E_DEVICE, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(W2V2_E_DEVICE, "hipEventElapsedTime failed");
    auto& t = p.totals[r.name];
    t.first += ms;
    t.second += 1;
    if (!p.names.count(r.name)) p.names[r.name] = r.name;
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.recs.clear();
  int i = 0;
  for (auto& kv : p.totals) {
    if (i < cap) {
      names[i] = p.names[kv.first];
      total_ms[i] = kv.second.first;
      launches[i] = kv.second.second;
    }
    ++i;
  }
  *n = i;
  p.totals.clear();
  return W2V2_OK;
}

}  // extern "C"
