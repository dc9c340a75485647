// Plain CPU oracle of one mixture-of-experts layer forward pass.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product imports, links or calls
// this file; only the tests, the smoke check and the benchmark's CPU-baseline
// leg do.  It shares no code, header, table or helper with the HIP library.
//
// Plain C++17, each token's arithmetic single-threaded (the *_threads drivers
// only hand contiguous token ranges of the same per-token code to std::threads):
// fp32 storage and fp32 element arithmetic, dot
// products accumulated in double and rounded once to fp32 (an order-free,
// near-correctly-rounded value of the fp32 dot product), no SIMD, no blocking,
// no reordering beyond what each step states.  Build with -ffp-contract=off.
//
// Sources (the pages are cited by title and section):
//   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
//           (localfirstai.eu, 5 October 2026)
//   [bench] "We Stopped the Kolibri Benchmark Before Scoring One Answer"
//           (localfirstai.eu, 9 October 2026)
//   [cache] "Kolibri-1 CPU dequant cache", vllm.cpp pull request 3488
//
// What the pages fix: a router scores every expert for every token in float32
// and sends the token to the top 6 by router score plus a per-expert selection
// bias, alongside one shared expert every token uses ([port] "The gate";
// "Taking it apart", part 1); a forced mode replays recorded expert choices
// ([bench] "The gate, forced"); the expert weights are FP8 and are decoded
// for compute ([cache], first paragraph); the expert layer is a gated-linear
// unit ([port] part 3).  What they leave open is read as follows (each reading
// is listed in the design notes):
//   * softmax over the k selected *unbiased* logits gives the weights; the
//     selection bias only ranks;
//   * ties in the selection score go to the lowest expert index;
//   * expert FFN = SwiGLU: y = W_down (silu(W_gate x) * (W_up x));
//   * FP8 weights: OCP E4M3 codes times one fp32 scale per 128x128 block;
//   * FP8 activations: per token and 128-element group, s = amax/448,
//     code = E4M3 round-to-nearest-even (saturating) of v/s, used as code*s;
//     the same for h before the down projection;
//   * combine: acc = shared; acc += w_j * y_j for slots j = 0..k-1 in fp32;
//     y = bf16 round-to-nearest-even of acc (fp32 output stays fp32);
//   * dispatch: a stable counting sort of the pairs p = t*k + j by expert.
//
// Parity pins (tests/test_oracle_pins.py): codecs vs torch's conversions,
// router vs a float64 BLAS matmul and exact integer sums, top-k vs a full
// stable sort, dispatch vs numpy's stable argsort, the FFN vs a float64
// textbook SwiGLU, exact-arithmetic FP8 cases, block-scale locality, the
// dense all-experts-masked restatement, and planted mutants that each pin
// must catch.  The activation-quantisation rule is fixed only by its own
// definition above ("parity unpinned" by the pages); the pins hold the one
// quantiser the forward runs (through oracle_expert_ffn_trace) to that
// definition bit for bit against torch's E4M3 conversion.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// ---- planted mutants (for the control tests; 0 = the correct oracle) -------
enum Mutant {
  MUT_NONE = 0,
  MUT_SELECT_UNBIASED = 1,   // rank by the logit even when a selection bias is given
  MUT_ROUTER_BF16 = 2,       // router weights rounded to bf16 before the dot product
  MUT_LOGITS_BF16 = 3,       // logits rounded to bf16
  MUT_TIE_HIGHEST = 4,       // ties go to the highest index
  MUT_SOFTMAX_ALL = 5,       // softmax over all experts, not renormalised over the top k
  MUT_NO_SHARED = 6,         // shared expert dropped
  MUT_SCALE_TRANSPOSED = 7,  // block-scale index transposed
  MUT_REVERSED_ORDER = 8,    // pairs of one expert in descending pair order
  MUT_NO_H_QUANT = 9,        // h not quantised before the down projection
  MUT_WEIGHTS_BIASED = 10,   // weights from the biased score instead of the logit
  MUT_SILU_SIGN = 11,        // silu(z) = z / (1 + exp(z))
  MUT_GATE_UP_SWAP = 12,     // silu applied to the up projection
  MUT_COMBINE_NO_WEIGHT = 13, // routed outputs added without their weights
  MUT_U4_NIBBLE_SWAP = 14,   // 4-bit codes: even columns read from the high nibble
  MUT_U4_NO_BIAS = 15,       // 4-bit groups: the bias term dropped
  MUT_U4_GROUP128 = 16,      // 4-bit groups: parameters indexed per 128 columns
  MUT_COMPARE_MIN_PAIR = 17, // routing comparison: a token's margin from its closest swapped pair
  MUT_COMPARE_UNBIASED = 18, // routing comparison: margins from the logits without the selection bias
  MUT_QUANT_RECIPROCAL = 19, // activation quantisation: v * (448 / amax) instead of v / (amax / 448)
  MUT_QUANT_TIES_AWAY = 20   // activation quantisation: E4M3 ties rounded away from zero
};
int g_mutant = MUT_NONE;

enum { ACT_F32 = 0, ACT_BF16 = 1 };
// W_FP8_A16: the same FP8 weights (codes and 128x128 block scales), with the
// activations entering both projections unquantised (W8A16): the CPU runtime of
// [cache] decodes the FP8 weights and runs its matmuls on the activations as
// they are.  Neither x nor h is quantised; everything else is as for W_FP8.
//
// W_U4: 4-bit weights, the analogue of the port's 4-bit (K4) build ([bench]
// "The gate, forced": an 8-bit and a 4-bit conversion, both run under MLX;
// "What this means if you want Kolibri on a Mac": the 4-bit build decodes
// faster).  The pages do not give the 4-bit format.  Reading: MLX's default
// affine group quantisation -- groups of 64 consecutive columns of a row,
// element value = scale * q + bias with q the unsigned 4-bit code and scale,
// bias bf16 per (row, group); codes two to a byte, the even column in the low
// nibble.  Activations and h stay unquantised, as in W_FP8_A16.
enum { W_F32 = 0, W_BF16 = 1, W_FP8 = 2, W_FP8_A16 = 3, W_U4 = 4 };
constexpr int kU4Group = 64;
enum { OK = 0, ERR_INVALID = -1, ERR_FORCED_INDEX = -5 };

// ---- number formats --------------------------------------------------------

float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t keep = u >> 16;
  uint32_t rest = u & 0xffffu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1;
  return (uint16_t)keep;
}

// OCP 8-bit floating point, E4M3 ("fn"): 1 sign bit, 4 exponent bits with
// bias 7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6;
// S.1111.111 is NaN; there is no infinity; the largest finite value is 448.
float e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 0xF;
  int m = c & 7;
  if (e == 15 && m == 7) return std::nanf("");
  float mag = (e == 0) ? std::ldexp((float)m / 8.0f, -6) : std::ldexp(1.0f + (float)m / 8.0f, e - 7);
  return sign ? -mag : mag;
}

// fp32 -> E4M3 code: nearest representable value, ties to the even code
// (even mantissa), magnitudes beyond 448 saturate to 448, NaN -> 0x7F.
// ties_away (planted-mutant control only): ties to the larger magnitude.
uint8_t e4m3_encode(float v, bool ties_away = false) {
  if (std::isnan(v)) return 0x7F;
  uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  float a = std::fabs(v);
  if (a >= 448.0f) return (uint8_t)(sign | 0x7E);
  // Non-negative codes 0x00..0x7E have increasing values; find the largest
  // code whose value is <= a by binary search, then pick the nearer of it and
  // the next code.
  int lo = 0, hi = 0x7E;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (e4m3_decode((uint8_t)mid) <= a) lo = mid; else hi = mid - 1;
  }
  int c = lo;
  if (c < 0x7E) {
    float below = e4m3_decode((uint8_t)c), above = e4m3_decode((uint8_t)(c + 1));
    float dlo = a - below, dhi = above - a;  // both exact: a and the grid are close
    if (dhi < dlo || (dhi == dlo && (ties_away || (c & 1)))) c += 1;
  }
  return (uint8_t)(sign | c);
}

// Dynamic quantisation of one group of n values, the oracle's only
// quantiser (the forward's x and h and the exported oracle_quant_groups all
// call it): s = amax/448 (one correctly rounded fp32 division), code_i =
// E4M3(v_i / s) rounded to nearest even and saturating; an all-zero group
// takes s = 1 and zero codes.  Returns s.
float quant_group(const float* v, int n, uint8_t* codes) {
  float amax = 0.0f;
  for (int i = 0; i < n; ++i) amax = std::fmax(amax, std::fabs(v[i]));
  if (!(amax > 0.0f)) {
    for (int i = 0; i < n; ++i) codes[i] = e4m3_encode(v[i]);  // zeros (signed)
    return 1.0f;
  }
  const float s = amax / 448.0f;
  const float r = 448.0f / amax;  // used only by the planted reciprocal mutant
  for (int i = 0; i < n; ++i) {
    const float q = g_mutant == MUT_QUANT_RECIPROCAL ? v[i] * r : v[i] / s;
    codes[i] = e4m3_encode(q, g_mutant == MUT_QUANT_TIES_AWAY);
  }
  return s;
}

// The values the next product sees: decode(code) * s, one fp32 multiply each.
void dequant_group(const uint8_t* codes, int n, float s, float* deq) {
  for (int i = 0; i < n; ++i) deq[i] = e4m3_decode(codes[i]) * s;
}

// What one expert FFN call quantised, for the pins (any pointer may be null):
// x codes [d] and scales [d/128], h before quantisation [F], h codes [F] and
// scales [F/128].
struct FfnTrace {
  uint8_t* x_codes;
  float* x_scales;
  float* h;
  uint8_t* h_codes;
  float* h_scales;
};

// ---- shapes and weights ----------------------------------------------------

struct Shape {
  int32_t T, d, E, k, F, Fs;
  int32_t act_dtype;  // ACT_F32 | ACT_BF16
  int32_t w_dtype;    // W_F32 | W_BF16 | W_FP8 | W_FP8_A16 | W_U4
};

struct Weights {
  const float* w_router;  // [E, d]
  const float* sel_bias;  // [E] or null
  const void* w_gate;     // [E, F, d]
  const void* w_up;       // [E, F, d]
  const void* w_down;     // [E, d, F]
  const float* s_gate;    // [E, F/128, d/128]   (FP8 only)
  const float* s_up;      // [E, F/128, d/128]
  const float* s_down;    // [E, d/128, F/128]
  const void* sh_gate;    // [Fs, d]
  const void* sh_up;      // [Fs, d]
  const void* sh_down;    // [d, Fs]
  const float* ss_gate;   // [Fs/128, d/128]
  const float* ss_up;
  const float* ss_down;   // [d/128, Fs/128]
  // W_U4: the s_* and ss_* pointers above hold bf16 group scales
  // [rows, cols/64] per matrix, and these the bf16 group biases
  const uint16_t* b_gate;   // [E, F, d/64]
  const uint16_t* b_up;     // [E, F, d/64]
  const uint16_t* b_down;   // [E, d, F/64]
  const uint16_t* sb_gate;  // [Fs, d/64]
  const uint16_t* sb_up;
  const uint16_t* sb_down;  // [d, Fs/64]
};

// One row-major weight matrix [rows, cols] in its storage format.
struct Mat {
  const void* data;
  const void* scale;    // FP8: fp32 [rows/128, cols/128]; U4: bf16 [rows, cols/64]
  const uint16_t* bias; // U4: bf16 [rows, cols/64]
  int rows, cols, w_dtype;
};

// The 256 E4M3 values, filled once from e4m3_decode (a lookup, same values).
const float* e4m3_table() {
  static float table[256];
  static bool ready = false;
  if (!ready) {
    for (int c = 0; c < 256; ++c) table[c] = e4m3_decode((uint8_t)c);
    ready = true;
  }
  return table;
}

// Element (r, c) of a weight matrix, decoded.  FP8: decode(code) * scale, one
// fp32 multiply.  U4: scale * q + bias, exact in double (a 4-bit integer times
// a bf16 value plus a bf16 value of similar size needs far fewer than 53 bits).
double mat_at(const Mat& m, int r, int c) {
  size_t i = (size_t)r * m.cols + c;
  if (m.w_dtype == W_F32) return ((const float*)m.data)[i];
  if (m.w_dtype == W_BF16) return bf16_to_f32(((const uint16_t*)m.data)[i]);
  if (m.w_dtype == W_U4) {
    const uint8_t byte = ((const uint8_t*)m.data)[i / 2];
    const bool high = (c % 2 == 1) != (g_mutant == MUT_U4_NIBBLE_SWAP);
    const int q = high ? byte >> 4 : byte & 0xF;
    const int group = g_mutant == MUT_U4_GROUP128 ? c / 128 : c / kU4Group;
    const size_t gi = (size_t)r * (m.cols / kU4Group) + group;
    const double scale = bf16_to_f32(((const uint16_t*)m.scale)[gi]);
    const double bias = g_mutant == MUT_U4_NO_BIAS ? 0.0 : bf16_to_f32(m.bias[gi]);
    return scale * q + bias;
  }
  int nrb = m.rows / 128, ncb = m.cols / 128;
  int si = (r / 128) * ncb + (c / 128);
  if (g_mutant == MUT_SCALE_TRANSPOSED) si = (c / 128) * nrb + (r / 128);
  return e4m3_table()[((const uint8_t*)m.data)[i]] * ((const float*)m.scale)[si];
}

float act_at(const Shape& s, const void* x, int t, int i) {
  size_t o = (size_t)t * s.d + i;
  return s.act_dtype == ACT_F32 ? ((const float*)x)[o] : bf16_to_f32(((const uint16_t*)x)[o]);
}

// out[r] = sum_c W[r, c] * v[c], accumulated in double, rounded once.
void matvec(const Mat& m, const float* v, float* out) {
  for (int r = 0; r < m.rows; ++r) {
    double acc = 0.0;
    for (int c = 0; c < m.cols; ++c) acc += mat_at(m, r, c) * (double)v[c];
    out[r] = (float)acc;
  }
}

float silu(float z) {
  if (g_mutant == MUT_SILU_SIGN) return z / (1.0f + std::exp(z));
  return z / (1.0f + std::exp(-z));
}

// One expert's SwiGLU FFN on one activation row already in compute form
// (FP8 mode: already quantised and dequantised).  expert = -1 is the shared
// expert.  [port] "The gate" (routed + shared experts), part 3 (a GLU layer).
void expert_ffn(const Shape& s, const Weights& w, int expert, const float* xin, float* y,
                const FfnTrace* trace = nullptr) {
  int F = expert < 0 ? s.Fs : s.F;
  Mat g, u, dn;
  if (expert < 0) {
    g = Mat{w.sh_gate, w.ss_gate, w.sb_gate, F, s.d, s.w_dtype};
    u = Mat{w.sh_up, w.ss_up, w.sb_up, F, s.d, s.w_dtype};
    dn = Mat{w.sh_down, w.ss_down, w.sb_down, s.d, F, s.w_dtype};
  } else if (s.w_dtype == W_U4) {
    const size_t cb = (size_t)F * s.d / 2;         // code bytes per matrix
    const size_t ng = (size_t)F * s.d / kU4Group;  // groups per matrix
    const uint16_t* sg = (const uint16_t*)w.s_gate;
    const uint16_t* su = (const uint16_t*)w.s_up;
    const uint16_t* sd = (const uint16_t*)w.s_down;
    g = Mat{(const char*)w.w_gate + expert * cb, sg + expert * ng, w.b_gate + expert * ng, F, s.d, s.w_dtype};
    u = Mat{(const char*)w.w_up + expert * cb, su + expert * ng, w.b_up + expert * ng, F, s.d, s.w_dtype};
    dn = Mat{(const char*)w.w_down + expert * cb, sd + expert * ng, w.b_down + expert * ng, s.d, F, s.w_dtype};
  } else {
    size_t esz = (size_t)F * s.d;
    size_t el = s.w_dtype == W_F32 ? 4 : (s.w_dtype == W_BF16 ? 2 : 1);
    size_t sgz = (size_t)(F / 128) * (s.d / 128);
    g = Mat{(const char*)w.w_gate + expert * esz * el, w.s_gate ? w.s_gate + expert * sgz : nullptr, nullptr, F, s.d,
            s.w_dtype};
    u = Mat{(const char*)w.w_up + expert * esz * el, w.s_up ? w.s_up + expert * sgz : nullptr, nullptr, F, s.d,
            s.w_dtype};
    dn = Mat{(const char*)w.w_down + expert * esz * el, w.s_down ? w.s_down + expert * sgz : nullptr, nullptr, s.d, F,
             s.w_dtype};
  }
  std::vector<float> gv(F), uv(F), h(F), hq(F);
  std::vector<uint8_t> hc(F);
  matvec(g, xin, gv.data());
  matvec(u, xin, uv.data());
  if (g_mutant == MUT_GATE_UP_SWAP) std::swap(gv, uv);
  for (int f = 0; f < F; ++f) h[f] = silu(gv[f]) * uv[f];
  if (trace && trace->h) std::memcpy(trace->h, h.data(), sizeof(float) * F);
  if (s.w_dtype == W_FP8 && g_mutant != MUT_NO_H_QUANT) {
    for (int f0 = 0; f0 < F; f0 += 128) {
      const float sc = quant_group(&h[f0], 128, &hc[f0]);
      dequant_group(&hc[f0], 128, sc, &hq[f0]);
      if (trace && trace->h_scales) trace->h_scales[f0 / 128] = sc;
    }
    if (trace && trace->h_codes) std::memcpy(trace->h_codes, hc.data(), F);
  } else {
    hq = h;
  }
  matvec(dn, hq.data(), y);
}

// Token t's activation row in compute form: fp32, and in FP8 mode quantised
// per 128-element group and dequantised.
void activation_row(const Shape& s, const void* x, int t, float* row, const FfnTrace* trace = nullptr) {
  std::vector<float> raw(s.d);
  for (int i = 0; i < s.d; ++i) raw[i] = act_at(s, x, t, i);
  if (s.w_dtype == W_FP8) {
    std::vector<uint8_t> codes(s.d);
    for (int i0 = 0; i0 < s.d; i0 += 128) {
      const float sc = quant_group(&raw[i0], 128, &codes[i0]);
      dequant_group(&codes[i0], 128, sc, &row[i0]);
      if (trace && trace->x_scales) trace->x_scales[i0 / 128] = sc;
    }
    if (trace && trace->x_codes) std::memcpy(trace->x_codes, codes.data(), s.d);
  } else {
    for (int i = 0; i < s.d; ++i) row[i] = raw[i];
  }
}

int check_shape(const Shape* s) {
  if (!s || s->T < 0 || s->d <= 0 || s->E <= 0 || s->k < 1 || s->k > s->E || s->F <= 0 || s->Fs < 0) return ERR_INVALID;
  if (s->w_dtype < W_F32 || s->w_dtype > W_U4) return ERR_INVALID;
  if ((s->w_dtype == W_FP8 || s->w_dtype == W_FP8_A16) && (s->d % 128 || s->F % 128 || s->Fs % 128))
    return ERR_INVALID;
  if (s->w_dtype == W_U4 && (s->d % kU4Group || s->F % kU4Group || s->Fs % kU4Group)) return ERR_INVALID;
  return OK;
}

// Router logits for token t: l[e] = sum_i x[t,i] * W_r[e,i] in fp32 terms,
// accumulated in double and rounded once.  [port] "The gate" (the router
// scores all 384 experts), part 3 (the router runs in float32); a bf16 router
// and bf16 logits are two of the planted bugs listed in "The gate".
void router_logits(const Shape& s, const Weights& w, const void* x, int t, float* l) {
  for (int e = 0; e < s.E; ++e) {
    double acc = 0.0;
    for (int i = 0; i < s.d; ++i) {
      float wr = w.w_router[(size_t)e * s.d + i];
      if (g_mutant == MUT_ROUTER_BF16) wr = bf16_to_f32(f32_to_bf16(wr));
      acc += (double)act_at(s, x, t, i) * (double)wr;
    }
    l[e] = (float)acc;
    if (g_mutant == MUT_LOGITS_BF16) l[e] = bf16_to_f32(f32_to_bf16(l[e]));
  }
}

// Routing weights over the k slots: softmax over the logits of the chosen
// experts (invalid slots, marked by a negative id, get weight 0 and take no
// part).  Z is summed in slot order.
void slot_weights(const Shape& s, const float* l, const float* score, const int32_t* idx, float* wout) {
  const float* src = (g_mutant == MUT_WEIGHTS_BIASED) ? score : l;
  if (g_mutant == MUT_SOFTMAX_ALL) {
    float m = -INFINITY;
    for (int e = 0; e < s.E; ++e) m = std::fmax(m, src[e]);
    float Z = 0.0f;
    for (int e = 0; e < s.E; ++e) Z = Z + std::exp(src[e] - m);
    for (int j = 0; j < s.k; ++j) wout[j] = idx[j] >= 0 ? std::exp(src[idx[j]] - m) / Z : 0.0f;
    return;
  }
  float m = -INFINITY;
  for (int j = 0; j < s.k; ++j)
    if (idx[j] >= 0) m = std::fmax(m, src[idx[j]]);
  std::vector<float> ex(s.k, 0.0f);
  float Z = 0.0f;
  for (int j = 0; j < s.k; ++j) {
    if (idx[j] < 0) continue;
    ex[j] = std::exp(src[idx[j]] - m);
    Z = Z + ex[j];
  }
  for (int j = 0; j < s.k; ++j) wout[j] = idx[j] >= 0 ? ex[j] / Z : 0.0f;
}

// Selection score: logit plus the per-expert selection bias ([port] part 1
// of "Taking it apart": experts are chosen by router score plus a per-expert
// selection bias).  NaN ranks below everything.
void selection_scores(const Shape& s, const Weights& w, const float* l, float* score) {
  for (int e = 0; e < s.E; ++e) {
    float v = l[e];
    if (w.sel_bias && g_mutant != MUT_SELECT_UNBIASED) v = v + w.sel_bias[e];
    if (std::isnan(v)) v = -INFINITY;
    score[e] = v;
  }
}

// Top-k by score, descending; equal scores go to the lower expert index.
void select_topk(const Shape& s, const float* score, int32_t* idx) {
  std::vector<char> taken(s.E, 0);
  for (int j = 0; j < s.k; ++j) {
    int best = -1;
    for (int e = 0; e < s.E; ++e) {
      if (taken[e]) continue;
      bool better;
      if (best < 0) better = true;
      else if (g_mutant == MUT_TIE_HIGHEST) better = score[e] >= score[best];
      else better = score[e] > score[best];
      if (better) best = e;
    }
    taken[best] = 1;
    idx[j] = best;
  }
}

const int32_t* token_ids(const int32_t* list, int n, std::vector<int32_t>& all) {
  if (list) return list;
  all.resize(n);
  for (int i = 0; i < n; ++i) all[i] = i;
  return all.data();
}

}  // namespace

extern "C" {

void oracle_set_mutant(int m) { g_mutant = m; }
int oracle_get_mutant(void) { return g_mutant; }

float oracle_e4m3_decode(uint8_t c) { return e4m3_decode(c); }
uint8_t oracle_e4m3_encode(float v) { return e4m3_encode(v); }
uint16_t oracle_f32_to_bf16(float v) { return f32_to_bf16(v); }

void oracle_e4m3_encode_array(const float* v, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(v[i]);
}
void oracle_f32_to_bf16_array(const float* v, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(v[i]);
}
// Dynamic group quantisation (s = amax/448): codes and scale per group of 128,
// through the same quant_group the forward uses for x and h.
void oracle_quant_groups(const float* v, int64_t n_groups, uint8_t* codes, float* scales) {
  for (int64_t g = 0; g < n_groups; ++g) scales[g] = quant_group(v + g * 128, 128, codes + g * 128);
}

// Free routing for the listed tokens (all T when token_list is null):
// logits [n,E], idx [n,k] in selection order, weights [n,k].
int oracle_route(const Shape* s, const Weights* w, const void* x, const int32_t* token_list, int32_t n_tokens,
                 float* logits, int32_t* idx, float* wts) {
  if (check_shape(s) != OK || !w || !w->w_router || !x) return ERR_INVALID;
  std::vector<int32_t> all;
  int n = token_list ? n_tokens : s->T;
  const int32_t* toks = token_ids(token_list, n, all);
  std::vector<float> l(s->E), score(s->E);
  for (int i = 0; i < n; ++i) {
    router_logits(*s, *w, x, toks[i], l.data());
    selection_scores(*s, *w, l.data(), score.data());
    select_topk(*s, score.data(), idx + (size_t)i * s->k);
    slot_weights(*s, l.data(), score.data(), idx + (size_t)i * s->k, wts + (size_t)i * s->k);
    if (logits) std::memcpy(logits + (size_t)i * s->E, l.data(), sizeof(float) * s->E);
  }
  return OK;
}

// Forced routing ([bench] "The gate, forced"): the recorded ids are used as
// given, in the given slot order; ids outside [0, E) make the call return
// ERR_FORCED_INDEX, their slot gets id -1 and weight 0 and the other slots
// are renormalised among themselves.  Duplicated ids are kept literally.
int oracle_route_forced(const Shape* s, const Weights* w, const void* x, const int32_t* forced, const int32_t* token_list,
                        int32_t n_tokens, float* logits, int32_t* idx, float* wts) {
  if (check_shape(s) != OK || !w || !w->w_router || !x || !forced) return ERR_INVALID;
  std::vector<int32_t> all;
  int n = token_list ? n_tokens : s->T;
  const int32_t* toks = token_ids(token_list, n, all);
  std::vector<float> l(s->E), score(s->E);
  int rc = OK;
  for (int i = 0; i < n; ++i) {
    int t = toks[i];
    router_logits(*s, *w, x, t, l.data());
    selection_scores(*s, *w, l.data(), score.data());
    int32_t* row = idx + (size_t)i * s->k;
    for (int j = 0; j < s->k; ++j) {
      int32_t e = forced[(size_t)t * s->k + j];
      if (e < 0 || e >= s->E) { rc = ERR_FORCED_INDEX; e = -1; }
      row[j] = e;
    }
    slot_weights(*s, l.data(), score.data(), row, wts + (size_t)i * s->k);
    if (logits) std::memcpy(logits + (size_t)i * s->E, l.data(), sizeof(float) * s->E);
  }
  return rc;
}

// Dispatch: stable counting sort of the pairs p = t*k + j by expert id.
// counts [E], offsets [E+1] (exclusive scan), perm [P] (perm[q] = p; slots past
// offsets[E] hold -1), inv_perm [P] (inv_perm[p] = q, -1 for invalid pairs).
// Within one expert the pairs ascend by p.  [port] part 3 and its update: the
// expert GEMM runs over (token, expert) rows sorted by expert.
int oracle_dispatch(int32_t T, int32_t k, int32_t E, const int32_t* idx, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* inv_perm) {
  if (T < 0 || k < 1 || E < 1 || (T > 0 && !idx)) return ERR_INVALID;
  int64_t P = (int64_t)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p)
    if (idx[p] >= 0 && idx[p] < E) counts[idx[p]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(E, 0);
  for (int64_t q = 0; q < P; ++q) perm[q] = -1;
  for (int64_t i = 0; i < P; ++i) {
    int64_t p = (g_mutant == MUT_REVERSED_ORDER) ? P - 1 - i : i;
    int32_t e = idx[p];
    if (e < 0 || e >= E) { inv_perm[p] = -1; continue; }
    int32_t q = offsets[e] + fill[e]++;
    perm[q] = (int32_t)p;
    inv_perm[p] = q;
  }
  return OK;
}

// Routing compared as a distribution ([port] "Taking it apart": after forcing
// the routing and comparing the rest closely, check the routing itself as a
// distribution; [bench] "The gate, forced": sigma is a layer's RMS router-
// logit error, and a disagreement is measured by the margin, in units of
// sigma, by which the reference made the choice the other side did not;
// [port] "What we couldn't explain": the disagreement count over (token,
// layer) pairs against an allowed rate).  Reading:
//   sigma^2 = mean over all T x E entries of (logits - ref_logits)^2;
//   a token disagrees when its set of chosen experts differs from the
//   reference's (ids outside [0, E) are ignored, slot order does not matter);
//   its margin is the largest s[e] - s[e'] over experts e the reference chose
//   and the other side did not, and e' the other way round, with s the
//   reference's selection score (ref logit plus the selection bias);
//   gap = margin / sigma (+inf when sigma = 0 and the margin is positive, 0
//   when both are 0); agreeing tokens get gap -1.
// Outputs: gap [T], sigma, the number of disagreeing tokens and the largest
// gap (-1 when none disagrees).  Sums in double, in token and expert order.
int oracle_route_compare(int32_t T, int32_t E, int32_t k, const float* logits, const float* ref_logits,
                         const float* sel_bias, const int32_t* idx, const int32_t* ref_idx, float* gap,
                         double* sigma, int32_t* n_disagree, float* max_gap) {
  if (T < 0 || E < 1 || k < 1 || (T > 0 && (!logits || !ref_logits || !idx || !ref_idx || !gap))) return ERR_INVALID;
  double ss = 0.0;
  for (int64_t i = 0; i < (int64_t)T * E; ++i) {
    const double dl = (double)logits[i] - (double)ref_logits[i];
    ss += dl * dl;
  }
  const double sg = T > 0 ? std::sqrt(ss / ((double)T * E)) : 0.0;
  auto chosen = [&](const int32_t* row, int e) {
    for (int j = 0; j < k; ++j)
      if (row[j] == e) return true;
    return false;
  };
  int32_t nd = 0;
  float mg = -1.0f;
  for (int t = 0; t < T; ++t) {
    const int32_t* a = idx + (size_t)t * k;
    const int32_t* r = ref_idx + (size_t)t * k;
    auto score = [&](int e) {
      float v = ref_logits[(size_t)t * E + e];
      if (sel_bias && g_mutant != MUT_COMPARE_UNBIASED) v = v + sel_bias[e];
      return (double)v;
    };
    bool differ = false;
    double margin = g_mutant == MUT_COMPARE_MIN_PAIR ? INFINITY : -INFINITY;
    for (int i = 0; i < k; ++i) {
      const int e = r[i];
      if (e < 0 || e >= E || chosen(a, e)) continue;  // e: the reference's choice only
      for (int j = 0; j < k; ++j) {
        const int f = a[j];
        if (f < 0 || f >= E || chosen(r, f)) continue;  // f: the other side's choice only
        differ = true;
        const double m = score(e) - score(f);
        margin = g_mutant == MUT_COMPARE_MIN_PAIR ? std::fmin(margin, m) : std::fmax(margin, m);
      }
    }
    // sets of different sizes (ignored ids) differ too, with no pair to measure
    for (int i = 0; i < k && !differ; ++i) {
      if (r[i] >= 0 && r[i] < E && !chosen(a, r[i])) differ = true;
      if (a[i] >= 0 && a[i] < E && !chosen(r, a[i])) differ = true;
    }
    if (!differ) {
      gap[t] = -1.0f;
      continue;
    }
    nd += 1;
    if (!std::isfinite(margin)) margin = 0.0;
    const double g = sg > 0.0 ? margin / sg : (margin > 0.0 ? INFINITY : 0.0);
    gap[t] = (float)g;
    mg = std::fmax(mg, gap[t]);
  }
  if (sigma) *sigma = sg;
  if (n_disagree) *n_disagree = nd;
  if (max_gap) *max_gap = mg;
  return OK;
}

// Layer output for the listed tokens given their routing (idx, wts are rows
// [n,k] aligned with the token list): acc = shared expert; acc += w_j * y_j in
// slot order (invalid slots, id < 0, skipped); y = bf16(acc) for bf16
// activations, acc for fp32.  y_f32 (optional) receives acc.
int oracle_forward(const Shape* s, const Weights* w, const void* x, const int32_t* idx, const float* wts,
                   const int32_t* token_list, int32_t n_tokens, void* y, float* y_f32) {
  if (check_shape(s) != OK || !w || !x || !idx || !wts) return ERR_INVALID;
  std::vector<int32_t> all;
  int n = token_list ? n_tokens : s->T;
  const int32_t* toks = token_ids(token_list, n, all);
  std::vector<float> xr(s->d), ye(s->d), acc(s->d);
  for (int i = 0; i < n; ++i) {
    activation_row(*s, x, toks[i], xr.data());
    for (int c = 0; c < s->d; ++c) acc[c] = 0.0f;
    if (s->Fs > 0 && g_mutant != MUT_NO_SHARED) {
      expert_ffn(*s, *w, -1, xr.data(), ye.data());
      for (int c = 0; c < s->d; ++c) acc[c] = ye[c];
    }
    for (int j = 0; j < s->k; ++j) {
      int32_t e = idx[(size_t)i * s->k + j];
      if (e < 0 || e >= s->E) continue;
      float wj = (g_mutant == MUT_COMBINE_NO_WEIGHT) ? 1.0f : wts[(size_t)i * s->k + j];
      expert_ffn(*s, *w, e, xr.data(), ye.data());
      for (int c = 0; c < s->d; ++c) {
        float prod = wj * ye[c];
        acc[c] = acc[c] + prod;
      }
    }
    for (int c = 0; c < s->d; ++c) {
      size_t o = (size_t)i * s->d + c;
      if (y) {
        if (s->act_dtype == ACT_F32) ((float*)y)[o] = acc[c];
        else ((uint16_t*)y)[o] = f32_to_bf16(acc[c]);
      }
      if (y_f32) y_f32[o] = acc[c];
    }
  }
  return OK;
}

// The same layer written as a dense sum over all experts with a selection
// mask: y = shared + sum_{e=0}^{E-1} [e chosen] * (sum of the chosen slots'
// weights for e) * E_e(x).  A restatement used to pin oracle_forward.
int oracle_forward_dense_masked(const Shape* s, const Weights* w, const void* x, const int32_t* idx, const float* wts,
                                float* y_f32) {
  if (check_shape(s) != OK || !w || !x || !idx || !wts || !y_f32) return ERR_INVALID;
  std::vector<float> xr(s->d), ye(s->d), acc(s->d);
  for (int t = 0; t < s->T; ++t) {
    activation_row(*s, x, t, xr.data());
    if (s->Fs > 0) expert_ffn(*s, *w, -1, xr.data(), ye.data());
    for (int c = 0; c < s->d; ++c) acc[c] = s->Fs > 0 ? ye[c] : 0.0f;
    for (int e = 0; e < s->E; ++e) {
      float mask_w = 0.0f;
      int chosen = 0;
      for (int j = 0; j < s->k; ++j)
        if (idx[(size_t)t * s->k + j] == e) { mask_w = mask_w + wts[(size_t)t * s->k + j]; chosen = 1; }
      expert_ffn(*s, *w, e, xr.data(), ye.data());  // every expert runs; the mask decides
      if (!chosen) continue;
      for (int c = 0; c < s->d; ++c) acc[c] = acc[c] + mask_w * ye[c];
    }
    for (int c = 0; c < s->d; ++c) y_f32[(size_t)t * s->d + c] = acc[c];
  }
  return OK;
}

// One expert on one token with what the call quantised (FP8 weights; the
// other modes leave the code and scale outputs untouched): the x codes [d] and
// scales [d/128] the forward uses, h before quantisation [F], its codes [F] and
// scales [F/128], the dequantised x row [d] and the output [d].  Null outputs
// are skipped.  The same activation_row and expert_ffn as oracle_forward.
int oracle_expert_ffn_trace(const Shape* s, const Weights* w, int32_t expert, const void* x, int32_t t,
                            uint8_t* x_codes, float* x_scales, float* h, uint8_t* h_codes, float* h_scales,
                            float* x_used, float* y) {
  if (check_shape(s) != OK || !w || !x || t < 0 || t >= s->T || expert < -1 || expert >= s->E || !y)
    return ERR_INVALID;
  const FfnTrace tr{x_codes, x_scales, h, h_codes, h_scales};
  std::vector<float> xr(s->d);
  activation_row(*s, x, t, xr.data(), &tr);
  if (x_used) std::memcpy(x_used, xr.data(), sizeof(float) * s->d);
  expert_ffn(*s, *w, expert, xr.data(), y, &tr);
  return OK;
}

// The same per-token oracle code on contiguous token ranges, one std::thread
// per range (the all-host-cores CPU baseline).  Each token's arithmetic is
// exactly that of the single-threaded call, so the outputs are bitwise equal
// to it.  n_threads < 1 means 1.
int oracle_route_threads(const Shape* s, const Weights* w, const void* x, const int32_t* token_list,
                         int32_t n_tokens, float* logits, int32_t* idx, float* wts, int32_t n_threads) {
  if (check_shape(s) != OK || !w || !w->w_router || !x) return ERR_INVALID;
  std::vector<int32_t> all;
  const int n = token_list ? n_tokens : s->T;
  const int32_t* toks = token_ids(token_list, n, all);
  const int nt = std::max(1, std::min<int>(n_threads, std::max(n, 1)));
  std::vector<std::thread> pool;
  std::vector<int> rcs(nt, OK);
  for (int i = 0; i < nt; ++i) {
    const int a = (int)((int64_t)n * i / nt), b = (int)((int64_t)n * (i + 1) / nt);
    pool.emplace_back([=, &rcs] {
      rcs[i] = oracle_route(s, w, x, toks + a, b - a, logits ? logits + (size_t)a * s->E : nullptr,
                            idx + (size_t)a * s->k, wts + (size_t)a * s->k);
    });
  }
  for (auto& th : pool) th.join();
  for (int rc : rcs)
    if (rc != OK) return rc;
  return OK;
}

int oracle_forward_threads(const Shape* s, const Weights* w, const void* x, const int32_t* idx, const float* wts,
                           const int32_t* token_list, int32_t n_tokens, void* y, float* y_f32, int32_t n_threads) {
  if (check_shape(s) != OK || !w || !x || !idx || !wts) return ERR_INVALID;
  e4m3_table();  // filled once here, before any thread reads it
  std::vector<int32_t> all;
  const int n = token_list ? n_tokens : s->T;
  const int32_t* toks = token_ids(token_list, n, all);
  const int nt = std::max(1, std::min<int>(n_threads, std::max(n, 1)));
  const size_t yel = s->act_dtype == ACT_F32 ? 4 : 2;
  std::vector<std::thread> pool;
  std::vector<int> rcs(nt, OK);
  for (int i = 0; i < nt; ++i) {
    const int a = (int)((int64_t)n * i / nt), b = (int)((int64_t)n * (i + 1) / nt);
    pool.emplace_back([=, &rcs] {
      rcs[i] = oracle_forward(s, w, x, idx + (size_t)a * s->k, wts + (size_t)a * s->k, toks + a, b - a,
                              y ? (char*)y + (size_t)a * s->d * yel : nullptr,
                              y_f32 ? y_f32 + (size_t)a * s->d : nullptr);
    });
  }
  for (auto& th : pool) th.join();
  for (int rc : rcs)
    if (rc != OK) return rc;
  return OK;
}

// One expert (expert = -1: the shared one) on one token, in compute form;
// also returns the activation row as the FFN sees it (FP8: dequantised).
int oracle_expert_ffn(const Shape* s, const Weights* w, int32_t expert, const void* x, int32_t t, float* x_used,
                      float* y) {
  if (check_shape(s) != OK || !w || !x || t < 0 || t >= s->T || expert < -1 || expert >= s->E) return ERR_INVALID;
  std::vector<float> xr(s->d);
  activation_row(*s, x, t, xr.data());
  if (x_used) std::memcpy(x_used, xr.data(), sizeof(float) * s->d);
  expert_ffn(*s, *w, expert, xr.data(), y);
  return OK;
}

}  // extern "C"
