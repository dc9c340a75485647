// Routing compared as a distribution (moe_route_compare).
//
// Pages cited by title and section:
//   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
//   [bench] "We Stopped the Kolibri Benchmark Before Scoring One Answer"
//
// [port] "Taking it apart" proposes to force the routing, compare the rest
// closely and check the routing itself as a distribution; [bench] "The gate,
// forced" measures a routing disagreement by the margin, in units of sigma (a
// layer's RMS router-logit error), by which the reference made the choice the
// other side did not; [port] "What we couldn't explain" counts the
// disagreeing (token, layer) pairs against an allowed rate.
//
// Three launches.  The first takes one wave per token: the token's sum of
// squared logit differences (double, lanes over experts, then a fixed
// butterfly), whether its expert set differs from the reference's, and the
// largest reference selection-score margin over the swapped experts.  The
// second is one block: sigma from the per-token sums in a fixed order.  The
// third takes one thread per token: its gap, and the number of disagreeing
// tokens and the largest gap through order-free atomics (an integer sum and a
// maximum).  Nothing depends on scheduling: the results are bitwise
// repeatable.
#include <limits.h>
#include <math.h>

#include "moe.h"
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int kCmpWaves = 4;

__global__ __launch_bounds__(kCmpWaves * 64) void route_compare_tokens_kernel(
    int T, int E, int k, const float* __restrict__ logits, const float* __restrict__ ref_logits,
    const float* __restrict__ bias, const int32_t* __restrict__ idx, const int32_t* __restrict__ ref_idx,
    double* __restrict__ sq, double* __restrict__ margin, int32_t* __restrict__ differ) {
  const int t = blockIdx.x * kCmpWaves + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  const float* la = logits + (size_t)t * E;
  const float* lr = ref_logits + (size_t)t * E;
  double s = 0.0;
  for (int e = lane; e < E; e += 64) {
    const double dl = (double)la[e] - (double)lr[e];
    s += dl * dl;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
  // Lane j < k holds slot j of both id rows.  The largest margin over pairs
  // (e only the reference chose, f only the other side chose) is the largest
  // such s[e] minus the smallest such s[f]: rounding is monotonic, so this
  // equals the largest of the pairwise differences in double.
  const bool slot = lane < k;
  const int a = slot ? idx[(size_t)t * k + lane] : -1;
  const int r = slot ? ref_idx[(size_t)t * k + lane] : -1;
  bool a_in_r = false, r_in_a = false;
  for (int i = 0; i < k; ++i) {
    const int ai = __shfl(a, i, kWave), ri = __shfl(r, i, kWave);
    a_in_r |= a == ri;
    r_in_a |= r == ai;
  }
  const bool r_only = r >= 0 && r < E && !r_in_a, a_only = a >= 0 && a < E && !a_in_r;
  auto score = [&](int e) { return (double)(bias ? lr[e] + bias[e] : lr[e]); };
  double hi = r_only ? score(r) : -INFINITY, lo = a_only ? score(a) : INFINITY;
#pragma unroll
  for (int o = 4; o >= 1; o >>= 1) {  // k <= 8: the slots sit in lanes 0..7
    hi = fmax(hi, __shfl_xor(hi, o, kWave));
    lo = fmin(lo, __shfl_xor(lo, o, kWave));
  }
  const bool diff = __any(r_only || a_only);
  if (lane == 0) {
    sq[t] = s;
    const double m = hi - lo;  // finite only when both sides have such an expert
    margin[t] = isfinite(m) ? m : 0.0;
    differ[t] = diff ? 1 : 0;
  }
}

constexpr int kCmpSigma = 1024;

// sigma from the per-token sums in a fixed order (per thread in token order,
// then a fixed butterfly per wave, then the waves in order); also resets the
// count and the largest gap for the gap launch.
__global__ __launch_bounds__(kCmpSigma) void route_compare_sigma_kernel(int T, int E, const double* __restrict__ sq,
                                                                        double* __restrict__ sigma,
                                                                        int32_t* __restrict__ n_differ,
                                                                        float* __restrict__ max_gap) {
  __shared__ double part[kCmpSigma / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double s = 0.0;
  for (int t = tid; t < T; t += kCmpSigma) s += sq[t];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
  if (lane == 0) part[wave] = s;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int w = 0; w < kCmpSigma / 64; ++w) tot += part[w];
    *sigma = sqrt(tot / ((double)T * E));
    *n_differ = 0;
    *max_gap = -1.0f;
  }
}

// One thread per token: gap = margin / sigma (or -1); the count and the
// largest gap per wave, then one atomic each (an integer sum and a maximum:
// the results do not depend on the order).
constexpr int kCmpGap = 256;

__global__ __launch_bounds__(kCmpGap) void route_compare_gap_kernel(int T, const double* __restrict__ margin,
                                                                    const int32_t* __restrict__ differ,
                                                                    const double* __restrict__ sigma,
                                                                    float* __restrict__ gap,
                                                                    int32_t* __restrict__ n_differ,
                                                                    float* __restrict__ max_gap) {
  const int t = blockIdx.x * kCmpGap + threadIdx.x, lane = threadIdx.x & 63;
  const double sg = *sigma;
  const bool d = t < T && differ[t];
  float g = -1.0f;
  if (d) {
    const double m = margin[t];
    g = (float)(sg > 0.0 ? m / sg : (m > 0.0 ? INFINITY : 0.0));
  }
  if (t < T) gap[t] = g;
  const int c = __popcll(__ballot(d));
  float gm = d ? g : -INFINITY;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o, kWave));
  if (lane == 0 && c > 0) {
    atomicAdd(n_differ, c);
    atomicMax(max_gap, gm);
  }
}

size_t route_compare_ws_bytes(int T) {
  auto a256 = [](size_t b) { return (b + 255) / 256 * 256; };
  return a256((size_t)T * 8) * 2 + a256((size_t)T * 4);
}

hipError_t launch_route_compare(int T, int E, int k, const float* logits, const float* ref_logits, const float* bias,
                                const int32_t* idx, const int32_t* ref_idx, float* gap, double* sigma,
                                int32_t* n_differ, float* max_gap, void* ws, hipStream_t st) {
  auto a256 = [](size_t b) { return (b + 255) / 256 * 256; };
  char* base = (char*)ws;
  double* sq = (double*)base;
  double* margin = (double*)(base + a256((size_t)T * 8));
  int32_t* differ = (int32_t*)(base + 2 * a256((size_t)T * 8));
  route_compare_tokens_kernel<<<(unsigned)((T + kCmpWaves - 1) / kCmpWaves), kCmpWaves * 64, 0, st>>>(
      T, E, k, logits, ref_logits, bias, idx, ref_idx, sq, margin, differ);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  route_compare_sigma_kernel<<<1, kCmpSigma, 0, st>>>(T, E, sq, sigma, n_differ, max_gap);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  route_compare_gap_kernel<<<(unsigned)((T + kCmpGap - 1) / kCmpGap), kCmpGap, 0, st>>>(T, margin, differ, sigma, gap,
                                                                                      n_differ, max_gap);
  return hipGetLastError();
}

}  // namespace moe
