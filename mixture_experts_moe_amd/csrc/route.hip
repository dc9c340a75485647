// Routing kernels: router logits, top-k selection with softmax weights, and the
// stable expert dispatch.
//
// Pages cited by title and section:
//   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
//   [bench] "We Stopped the Kolibri Benchmark Before Scoring One Answer"
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits l[t][e] = sum_i x[t][i] * W_r[e][i], fp32 multiply-add
// ([port] "The gate": every expert is scored for every token; part 3: the
// router stays in float32).  Tiles of TT tokens x TE experts; the K dimension
// is staged through LDS in chunks of 32; each of the 256 threads owns a
// (TT/16) x (TE/16) register tile.
// ---------------------------------------------------------------------------
template <int TT, int TE, bool XBF16>
__global__ __launch_bounds__(256) void router_logits_kernel(const void* __restrict__ x, const float* __restrict__ W,
                                                             float* __restrict__ logits, int T, int d, int E,
                                                             int32_t* __restrict__ status) {
  constexpr int KC = 32, MT = TT / 16, ME = TE / 16;
  __shared__ float xs[KC][TT + 1];
  __shared__ float ws[KC][TE + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
  if (status && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *status = 0;
  float acc[MT][ME];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < ME; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < d; k0 += KC) {
    for (int i = tid; i < TT * KC; i += 256) {
      const int r = i / KC, c = i % KC, t = t0 + r;
      float v = 0.f;
      if (t < T) {
        const size_t o = (size_t)t * d + k0 + c;
        v = XBF16 ? bf16_to_f32(((const uint16_t*)x)[o]) : ((const float*)x)[o];
      }
      xs[c][r] = v;
    }
    for (int i = tid; i < TE * KC; i += 256) {
      const int r = i / KC, c = i % KC, e = e0 + r;
      ws[c][r] = e < E ? W[(size_t)e * d + k0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < KC; ++k) {
      float a[MT], b[ME];
#pragma unroll
      for (int i = 0; i < MT; ++i) a[i] = xs[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < ME; ++j) b[j] = ws[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < ME; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < ME; ++j) {
      const int t = t0 + ty + 16 * i, e = e0 + tx + 16 * j;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j];
    }
}

// Order-preserving 64-bit key: high word the selection score mapped to an
// unsigned order (NaN ranks as -inf, -0 equals +0), low word ~e so that the
// lower expert index wins among equal scores.  0 is below every real key.
__device__ __forceinline__ uint64_t select_key(float s, int e) {
  if (s != s) s = -INFINITY;
  if (s == 0.0f) s = 0.0f;
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)e);
}

// ---------------------------------------------------------------------------
// Free top-k: one wave per token.  Lane l holds candidates e = l + 64 j.  The
// selection score is logit + bias ([port] part 1 of "Taking it apart": router
// score plus a per-expert selection bias); k rounds of a wave-wide maximum of
// the 64-bit key pick the experts in descending score, lowest index on ties.
// The weights are the softmax over the chosen experts' unbiased logits
// (normalisation sum in slot order).
// ---------------------------------------------------------------------------
template <int J>
__global__ __launch_bounds__(256) void topk_free_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                                                         int T, int E, int k, int32_t* __restrict__ idx,
                                                         float* __restrict__ wout) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float lv[J];
  uint64_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    lv[j] = 0.f;
    key[j] = 0;
    if (e < E) {
      const float l = logits[(size_t)t * E + e];
      lv[j] = l;
      key[j] = select_key(bias ? l + bias[e] : l, e);
    }
  }
  int sel[8];
  float sl[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    sel[r] = 0;
    sl[r] = 0.f;
    if (r < k) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) best = key[j] > best ? key[j] : best;
      best = wave_max_u64(best);
      const int e = (int)(~(uint32_t)best);
      float mine = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (lane + 64 * j == e) {
          key[j] = 0;
          mine = lv[j];
        }
      sel[r] = e;
      sl[r] = __shfl(mine, e & 63, kWave);
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < k) m = fmaxf(m, sl[r]);
  float ex[8], Z = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    ex[r] = 0.f;
    if (r < k) {
      ex[r] = expf(sl[r] - m);
      Z = Z + ex[r];
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < k && lane == r) {
      idx[(size_t)t * k + r] = sel[r];
      wout[(size_t)t * k + r] = ex[r] / Z;
    }
}

// ---------------------------------------------------------------------------
// Forced top-k ([bench] "The gate, forced": recorded choices replayed at every
// position): one thread per token; the given ids keep their slot order; an id
// outside [0, E) flags the status word, becomes -1 with weight 0, and the
// remaining slots are renormalised among themselves.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void topk_forced_kernel(const float* __restrict__ logits,
                                                           const int32_t* __restrict__ forced, int T, int E, int k,
                                                           int32_t* __restrict__ idx, float* __restrict__ wout,
                                                           int32_t* __restrict__ status) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int sel[8];
  float sl[8];
  bool bad = false;
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    sel[r] = -1;
    sl[r] = 0.f;
    if (r < k) {
      const int e = forced[(size_t)t * k + r];
      if (e >= 0 && e < E) {
        sel[r] = e;
        sl[r] = logits[(size_t)t * E + e];
        m = fmaxf(m, sl[r]);
      } else {
        bad = true;
      }
    }
  }
  float ex[8], Z = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    ex[r] = 0.f;
    if (r < k && sel[r] >= 0) {
      ex[r] = expf(sl[r] - m);
      Z = Z + ex[r];
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r)
    if (r < k) {
      idx[(size_t)t * k + r] = sel[r];
      wout[(size_t)t * k + r] = sel[r] >= 0 ? ex[r] / Z : 0.f;
    }
  if (bad) *status = -5;  // MOE_ERR_FORCED_INDEX; every writer stores the same value
}

// ---------------------------------------------------------------------------
// Dispatch: a stable counting sort of the pairs p = t*k + j by expert
// ([port] part 3 and its update: the expert matmul consumes (token, expert)
// rows sorted by expert).  Deterministic in three launches:
//   1. per chunk of 256 pairs: LDS-atomic histogram (order-free integer counts)
//      and each pair's rank among the equal ids before it in the chunk;
//   2. one block: per expert, an exclusive scan of the chunk histograms in
//      chunk order, the expert totals, and their exclusive scan (offsets);
//   3. per pair: q = offsets[e] + (pairs of e in earlier chunks) + rank.
// ---------------------------------------------------------------------------
constexpr int kChunk = 256;

__global__ __launch_bounds__(256) void dispatch_local_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                              int32_t* __restrict__ chunk_hist,
                                                              int32_t* __restrict__ local_rank) {
  __shared__ int32_t hist[kMaxExperts];
  __shared__ int32_t ids[kChunk];
  const int tid = threadIdx.x, c = blockIdx.x, p = c * kChunk + tid;
  for (int i = tid; i < E; i += kChunk) hist[i] = 0;
  int e = -1;
  if (p < P) {
    e = idx[p];
    if (e < 0 || e >= E) e = -1;
  }
  ids[tid] = e;
  __syncthreads();
  if (e >= 0) atomicAdd(&hist[e], 1);
  int r = 0;
  for (int j = 0; j < tid; ++j) r += (ids[j] == e);
  if (p < P) local_rank[p] = r;
  __syncthreads();
  for (int i = tid; i < E; i += kChunk) chunk_hist[(size_t)c * E + i] = hist[i];
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t* __restrict__ chunk_hist, int n_chunks, int E,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets) {
  __shared__ int32_t tmp[17];
  const int e = threadIdx.x;  // E <= kMaxExperts <= 1024
  int run = 0;
  if (e < E) {
    for (int c = 0; c < n_chunks; ++c) {
      const int h = chunk_hist[(size_t)c * E + e];
      chunk_hist[(size_t)c * E + e] = run;
      run += h;
    }
    counts[e] = run;
  }
  int total;
  const int ex = block1024_excl_scan(e < E ? run : 0, tmp, &total);
  if (e < E) offsets[e] = ex;
  if (e == 0) offsets[E] = total;
}

__global__ __launch_bounds__(256) void dispatch_place_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                              const int32_t* __restrict__ chunk_prefix,
                                                              const int32_t* __restrict__ local_rank,
                                                              const int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv_perm) {
  const int c = blockIdx.x, p = c * kChunk + threadIdx.x;
  if (p >= P) return;
  const int e = idx[p];
  if (e >= 0 && e < E) {
    const int q = offsets[e] + chunk_prefix[(size_t)c * E + e] + local_rank[p];
    perm[q] = p;
    inv_perm[p] = q;
  } else {
    inv_perm[p] = -1;
  }
  if (p >= offsets[E]) perm[p] = -1;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_router_logits(const void* x, bool x_bf16, const float* W, float* logits, int T, int d, int E,
                                int32_t* status, hipStream_t st) {
  if (T >= 256) {
    dim3 grid((T + 63) / 64, (E + 63) / 64);
    if (x_bf16) router_logits_kernel<64, 64, true><<<grid, 256, 0, st>>>(x, W, logits, T, d, E, status);
    else router_logits_kernel<64, 64, false><<<grid, 256, 0, st>>>(x, W, logits, T, d, E, status);
  } else {
    dim3 grid((T + 31) / 32, (E + 15) / 16);
    if (x_bf16) router_logits_kernel<32, 16, true><<<grid, 256, 0, st>>>(x, W, logits, T, d, E, status);
    else router_logits_kernel<32, 16, false><<<grid, 256, 0, st>>>(x, W, logits, T, d, E, status);
  }
  return hipGetLastError();
}

hipError_t launch_topk_free(const float* logits, const float* bias, int T, int E, int k, int32_t* idx, float* w,
                            hipStream_t st) {
  const int J = (E + 63) / 64;
  dim3 grid((T + 3) / 4);
#define MOE_TOPK_CASE(n) \
  case n: topk_free_kernel<n><<<grid, 256, 0, st>>>(logits, bias, T, E, k, idx, w); break;
  switch (J) {
    MOE_TOPK_CASE(1) MOE_TOPK_CASE(2) MOE_TOPK_CASE(3) MOE_TOPK_CASE(4) MOE_TOPK_CASE(5) MOE_TOPK_CASE(6)
    MOE_TOPK_CASE(7) MOE_TOPK_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

hipError_t launch_topk_forced(const float* logits, const int32_t* forced, int T, int E, int k, int32_t* idx, float* w,
                              int32_t* status, hipStream_t st) {
  topk_forced_kernel<<<(T + 255) / 256, 256, 0, st>>>(logits, forced, T, E, k, idx, w, status);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* idx, int P, int E, int32_t* chunk_hist, int32_t* local_rank,
                           int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, hipStream_t st) {
  const int n_chunks = (P + kChunk - 1) / kChunk;
  dispatch_local_kernel<<<n_chunks, kChunk, 0, st>>>(idx, P, E, chunk_hist, local_rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dispatch_scan_kernel<<<1, 1024, 0, st>>>(chunk_hist, n_chunks, E, counts, offsets);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dispatch_place_kernel<<<n_chunks, kChunk, 0, st>>>(idx, P, E, chunk_hist, local_rank, offsets, perm, inv_perm);
  return hipGetLastError();
}

size_t dispatch_chunk_hist_ints(int P, int E) { return (size_t)((P + kChunk - 1) / kChunk) * E; }

}  // namespace moe
