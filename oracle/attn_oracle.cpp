// Plain CPU oracle of the attention ops next to the mixture-of-experts layer:
// rotary position encoding and causal attention over a sliding window or the
// whole context.
//
// TEST INFRASTRUCTURE ONLY.  Nothing in the product imports, links or calls
// this file; only the tests and the benchmark's CPU-baseline leg do.  It
// shares no code, header, table or helper with the HIP library.
//
// Plain single-threaded C++17, every value in double, rounded once at the end.
//
// Sources (cited by title and section):
//   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
//           "The gate": forty layers attend over a sliding window of 513 tokens
//           and mark position with rotary position encoding; every fifth layer
//           attends over the whole context with no positional encoding; "a
//           window one token short" is one of the planted bugs.  "Taking it
//           apart", part 2: each pair of dimensions of a query or key is rotated
//           by the token's position times a fixed frequency, the textbook
//           frequency being 1/theta^(2j/D).
//   [bench] "We Stopped the Kolibri Benchmark Before Scoring One Answer",
//           "The pilot that ran out of buffers, not memory": the same layout
//           (forty sliding-window RoPE layers, ten whole-context NoPE layers).
//
// Readings where the pages are silent: the rotated pairs are (j, j + D/2)
// (the split-halves form), theta is an input, scores are q.k / sqrt(D),
// softmax over the attended keys, query heads share key/value heads in
// consecutive groups (head h uses key/value head h / (Hq/Hkv)), and a window
// of W lets a query at position p see keys at positions p-W+1 .. p.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

enum { OK = 0, ERR_INVALID = -1 };
enum { MUT_NONE = 0, MUT_WINDOW_SHORT = 1, MUT_ROPE_INTERLEAVED = 2, MUT_NO_SCALE = 3, MUT_ROPE_SIGN = 4 };
int g_mutant = MUT_NONE;

double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// double -> bf16: round to nearest, ties to even, via the exact float value
// when it is representable, else the double's own bits (no double rounding:
// the comparison is done on the double directly).
uint16_t double_to_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  float f = (float)v;  // candidates bracket v within one float ulp
  uint32_t u;
  std::memcpy(&u, &f, 4);
  uint32_t lo = u & 0xFFFF0000u;          // truncated toward zero (magnitude)
  uint32_t hi = lo + 0x10000u;            // next bf16 away from zero
  float flo, fhi;
  std::memcpy(&flo, &lo, 4);
  std::memcpy(&fhi, &hi, 4);
  const double dlo = std::fabs(v - (double)flo), dhi = std::fabs((double)fhi - v);
  if (dlo < dhi) return (uint16_t)(lo >> 16);
  if (dhi < dlo) return (uint16_t)(hi >> 16);
  return (uint16_t)(((lo >> 16) & 1) ? (hi >> 16) : (lo >> 16));
}

}  // namespace

extern "C" {

void attn_oracle_set_mutant(int m) { g_mutant = m; }

// Rotary position encoding of x [T][H][D] (bf16 bits), in place: token t at
// position pos0 + t; for j < D/2 the pair (x_j, x_{j+D/2}) is rotated by the
// angle (pos0 + t) / theta^(2j/D):  x_j' = x_j cos - x_{j+D/2} sin,
// x_{j+D/2}' = x_j sin + x_{j+D/2} cos; results rounded to bf16.
int attn_oracle_rope(int32_t T, int32_t H, int32_t D, int32_t pos0, double theta, uint16_t* x) {
  if (T < 0 || H < 1 || D < 2 || D % 2 || pos0 < 0 || !(theta > 1.0) || (T > 0 && !x)) return ERR_INVALID;
  const int half = D / 2;
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      uint16_t* row = x + ((size_t)t * H + h) * D;
      std::vector<double> v(D);
      for (int i = 0; i < D; ++i) v[i] = bf16_to_double(row[i]);
      for (int j = 0; j < half; ++j) {
        const double ang = (double)(pos0 + t) / std::pow(theta, 2.0 * j / D);
        const double c = std::cos(ang), s = g_mutant == MUT_ROPE_SIGN ? -std::sin(ang) : std::sin(ang);
        const int a = g_mutant == MUT_ROPE_INTERLEAVED ? 2 * j : j;
        const int b = g_mutant == MUT_ROPE_INTERLEAVED ? 2 * j + 1 : j + half;
        const double xa = v[a], xb = v[b];
        row[a] = double_to_bf16(xa * c - xb * s);
        row[b] = double_to_bf16(xa * s + xb * c);
      }
    }
  return OK;
}

// Causal attention.  q [Tq][Hq][D], k and v [Tk][Hkv][D] (bf16 bits); query i
// sits at position q_pos0 + i, key j at position j.  A query at position p
// attends the keys j <= p with p - j < window (window 0: no limit); scores
// s_j = q.k_j / sqrt(D); o = sum_j softmax(s)_j v_j, written as fp32
// [Tq][Hq][D].  Needs q_pos0 + Tq <= Tk (every query sees at least itself).
int attn_oracle_attention(int32_t Tq, int32_t Tk, int32_t Hq, int32_t Hkv, int32_t D, int32_t q_pos0,
                          int32_t window, const uint16_t* q, const uint16_t* k, const uint16_t* v, float* o) {
  if (Tq < 0 || Tk < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || q_pos0 < 0 || window < 0 ||
      (int64_t)q_pos0 + Tq > Tk || (Tq > 0 && (!q || !k || !v || !o)))
    return ERR_INVALID;
  const int G = Hq / Hkv;
  const int W = window > 0 && g_mutant == MUT_WINDOW_SHORT ? window - 1 : window;
  const double scale = g_mutant == MUT_NO_SCALE ? 1.0 : 1.0 / std::sqrt((double)D);
  std::vector<double> s(Tk), acc(D);
  for (int i = 0; i < Tq; ++i) {
    const int p = q_pos0 + i;
    const int j0 = W > 0 ? (p - W + 1 > 0 ? p - W + 1 : 0) : 0;
    for (int h = 0; h < Hq; ++h) {
      const int g = h / G;
      const uint16_t* qr = q + ((size_t)i * Hq + h) * D;
      double m = -INFINITY;
      for (int j = j0; j <= p; ++j) {
        const uint16_t* kr = k + ((size_t)j * Hkv + g) * D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += bf16_to_double(qr[d]) * bf16_to_double(kr[d]);
        s[j] = dot * scale;
        m = std::fmax(m, s[j]);
      }
      double l = 0.0;
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      for (int j = j0; j <= p; ++j) {
        const double e = std::exp(s[j] - m);
        l += e;
        const uint16_t* vr = v + ((size_t)j * Hkv + g) * D;
        for (int d = 0; d < D; ++d) acc[d] += e * bf16_to_double(vr[d]);
      }
      float* orow = o + ((size_t)i * Hq + h) * D;
      for (int d = 0; d < D; ++d) orow[d] = (float)(acc[d] / l);
    }
  }
  return OK;
}

}  // extern "C"
