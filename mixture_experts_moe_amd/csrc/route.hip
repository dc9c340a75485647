// Routing kernels: router logits, top-k selection with softmax weights, and the
// stable expert dispatch.
//
// Pages cited by title and section:
//   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
//   [bench] "We Stopped the Kolibri Benchmark Before Scoring One Answer"
//
// Launch sequence of one routing call.  The router (bf16 activations) is split
// along K at every T: one block per (16 experts, K slice, token tile) writes
// partial dot products, which top-k adds in slice order, so a token's logits
// (and so its experts) never depend on T or on the batch around it.
// Short inputs (T * k <= 1024 pairs, e.g. a decode batch), three launches:
//   1. router partial sums;
//   2. top-k, one wave per token: adds the slices, selects, softmax weights;
//   3. the whole counting sort in one block.
// Long inputs, four launches:
//   1. router partial sums;
//   2. top-k per chunk of tokens, and the chunk's share of the dispatch;
//   3. scan of the chunk histograms into counts and offsets;
//   4. placement of every pair.
#include "moe_device.h"
#include "moe_kernels.h"
#include "moe_plan.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits for bf16 activations, on the matrix cores at fp32 accuracy
// ([port] "The gate": every expert is scored for every token; part 3 of "Taking
// it apart": the router stays in float32, a bf16 router being one of the
// planted bugs).  Each fp32 router weight is split exactly into three bf16
// terms, w = hi + mid + lo (each term is the bf16 rounding of what the previous
// ones leave, and the last remainder has at most 8 significant bits); x is
// already bf16, so every product x*hi, x*mid, x*lo is exact in fp32 and the
// matrix core accumulates them in fp32.  The result is an fp32 dot product of
// x and W_r; only the summation order differs from a scalar loop.
// ---------------------------------------------------------------------------

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// The split of two weights at once: each bf16 rounding (to nearest even) is
// one packed conversion of the pair, the remainders exact fp32 differences.
// Results as packed pairs (element 0 in the low half).
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const v2f w = {a, b};
  const v2bf h = __builtin_convertvector(w, v2bf);
  const v2f r1 = w - __builtin_convertvector(h, v2f);
  const v2bf m = __builtin_convertvector(r1, v2bf);
  const v2f r2 = r1 - __builtin_convertvector(m, v2f);
  hi = __builtin_bit_cast(uint32_t, h);
  mid = __builtin_bit_cast(uint32_t, m);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, v2bf));
}

__device__ __forceinline__ void split3_bf16(const float (&w)[8], v8bf& hi, v8bf& mid, v8bf& lo) {
  v4i h, m, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t a, b, c;
    split3_pair(w[2 * j], w[2 * j + 1], a, b, c);
    h[j] = (int)a;
    m[j] = (int)b;
    l[j] = (int)c;
  }
  hi = __builtin_bit_cast(v8bf, h);
  mid = __builtin_bit_cast(v8bf, m);
  lo = __builtin_bit_cast(v8bf, l);
}

// Router partial logits for short inputs, split along K: block (16 experts,
// K slice ks of 4*32*NS, tile of 16*NC tokens) writes its slice's dot products
// to part[ks][t][e]; the top-k kernel adds the slices in slice order.  Same
// exact three-way split of the fp32 weights as above; each of the 4 waves takes
// a quarter of the slice and the quarters are added through LDS in wave order.
template <int NC, int NS>
__global__ __launch_bounds__(256) void router_split_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ W, float* __restrict__ part,
                                                           int T, int d, int E, int32_t* __restrict__ status) {
  constexpr int KW = 32 * NS;  // K per wave
  __shared__ float red[4][NC][4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lk = (lane >> 4) * 8;
  const int e0 = blockIdx.x * 16, ks = blockIdx.y, t0 = blockIdx.z * 16 * NC;
  const int k0 = (ks * 4 + wave) * KW;
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *status = 0;
  const int e = e0 + lr;
  const bool ev = e < E;
  const float* wp = W + (size_t)(ev ? e : E - 1) * d + k0 + lk;
  float4 wa[NS][2];
  v4i xb[NS][NC];
  bool tv[NC];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    wa[u][0] = *(const float4*)(wp + 32 * u);
    wa[u][1] = *(const float4*)(wp + 32 * u + 4);
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = t0 + c * 16 + lr;
    tv[c] = t < T;
    const uint16_t* xp = x + (size_t)(tv[c] ? t : T - 1) * d + k0 + lk;
#pragma unroll
    for (int u = 0; u < NS; ++u) xb[u][c] = *(const v4i*)(xp + 32 * u);
  }
  v4f acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    float wv[8] = {wa[u][0].x, wa[u][0].y, wa[u][0].z, wa[u][0].w, wa[u][1].x, wa[u][1].y, wa[u][1].z, wa[u][1].w};
    if (!ev) {
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = 0.f;
    }
    v8bf hi, mid, lo;
    split3_bf16(wv, hi, mid, lo);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const v8bf b = tv[c] ? __builtin_bit_cast(v8bf, xb[u][c]) : v8bf{};
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, b, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[c], 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][c][i][lane] = acc[c][i];
  __syncthreads();
  for (int o = threadIdx.x; o < NC * 256; o += 256) {
    const int c = o / 256, i = (o / 64) & 3, l = o & 63;
    const float v = ((red[0][c][i][l] + red[1][c][i][l]) + red[2][c][i][l]) + red[3][c][i][l];
    const int t = t0 + c * 16 + (l & 15), ee = e0 + 4 * (l >> 4) + i;
    if (t < T && ee < E) part[((size_t)ks * T + t) * E + ee] = v;
  }
}

// ---------------------------------------------------------------------------
// Router partial logits for long inputs (bf16 x): tiles of 64 tokens x 64
// experts over one half of the K range (blockIdx.z), NW waves: 8 waves of 32
// tokens x 16 experts for 64-deep chunks, 4 waves of 32 x 32 for 32-deep ones
// (so every thread stages one piece of x and two of W per chunk); the
// halves split at slice gsl (256-deep slices, the same boundary the top-k
// kernel uses; one half when there is a single slice).  Both operands are staged in LDS per chunk of 32*NS K (two LDS
// buffers, the chunk after next prefetched into registers); the fp32 weights
// are split into their three exact bf16 terms while staged.  Sum order per
// logit: per chunk a chain of 3*NS products from zero, four chunks added in
// order into a slice, the half's slices added in order -- the K-split kernel's
// order, so both kernels give the same logits bit for bit.
// ---------------------------------------------------------------------------
template <int NS, int NW>
__global__ __launch_bounds__(NW * 64) void router_tile_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ W, float* __restrict__ part,
                                                              int T, int d, int E, int gsl,
                                                              int32_t* __restrict__ status) {
  constexpr int TT = 64, TE = 64, KC = 32 * NS;  // tile, K per chunk
  constexpr int NT = NW * 64;                      // threads
  constexpr int IT = 8 / NW;                       // 16-expert tiles per wave (waves: 2 along tokens)
  constexpr int XS = KC * 2 + 16;                  // LDS row stride (bytes), padded
  constexpr int XP = TT * KC / 8;                  // x pieces (8 bf16) per chunk
  constexpr int WP = TE * KC / 4;                  // W pieces (4 fp32) per chunk
  constexpr int PX = XP / NT, PW = WP / NT;        // per thread
  static_assert(PX * NT == XP && PW * NT == WP && IT * 16 * (NW / 2) == TE, "tile shape");
  __shared__ __align__(16) uint8_t xs[2][TT * XS];
  __shared__ __align__(16) uint8_t wsm[2][3 * TE * XS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, kg = lane >> 4;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE, half = blockIdx.z;
  const int wt = wave & 1, we = wave >> 1;
  if (blockIdx.x == 0 && blockIdx.y == 0 && half == 0 && tid == 0) *status = 0;
  constexpr int cps = 4;  // chunks per slice (a slice is 4*KC deep, as in the K-split kernel)
  const int c0 = half ? gsl * cps : 0, c1 = half ? d / KC : gsl * cps;  // a multiple of 4 chunks, >= 4
  struct Pre {
    v4i xv[PX];
    float4 wv[PW];
  };
  auto fetch = [&](int ch, Pre& p) {
    const int k0 = ch * KC;
#pragma unroll
    for (int u = 0; u < PX; ++u) {
      const int i = tid + u * NT, r = i / (KC / 8), c = i % (KC / 8), t = min(t0 + r, T - 1);
      p.xv[u] = *(const v4i*)(x + (size_t)t * d + k0 + c * 8);
    }
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int i = tid + u * NT, r = i / (KC / 4), c = i % (KC / 4), e = min(e0 + r, E - 1);
      p.wv[u] = *(const float4*)(W + (size_t)e * d + k0 + c * 4);
    }
  };
  auto store = [&](int buf, const Pre& p) {
    // Rows past T or E hold a clamped copy of the last row (fetch); the
    // outputs they feed are never stored, so they need no zeroing.
#pragma unroll
    for (int u = 0; u < PX; ++u) {
      const int i = tid + u * NT, r = i / (KC / 8), c = i % (KC / 8);
      *(v4i*)(xs[buf] + r * XS + c * 16) = p.xv[u];
    }
#pragma unroll
    for (int u = 0; u < PW; ++u) {
      const int i = tid + u * NT, r = i / (KC / 4), c = i % (KC / 4);
      uint2 pk[3];
      split3_pair(p.wv[u].x, p.wv[u].y, pk[0].x, pk[1].x, pk[2].x);
      split3_pair(p.wv[u].z, p.wv[u].w, pk[0].y, pk[1].y, pk[2].y);
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) *(uint2*)(wsm[buf] + (sp * TE + r) * XS + c * 8) = pk[sp];
    }
  };
  v4f tot[IT][2], sl[IT][2];
#pragma unroll
  for (int i = 0; i < IT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) tot[i][j] = sl[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, int ch) {
    v4f cc[IT][2];
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) cc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NS; ++u) {  // 32-deep steps; lane holds K = 32u + 8*kg + [0, 8)
      v8bf b[2], a[3][IT];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const v8bf*)(xs[buf] + (wt * 32 + j * 16 + lr) * XS + u * 64 + kg * 16);
#pragma unroll
      for (int sp = 0; sp < 3; ++sp)
#pragma unroll
        for (int i = 0; i < IT; ++i)
          a[sp][i] = *(const v8bf*)(wsm[buf] + (sp * TE + we * 16 * IT + i * 16 + lr) * XS + u * 64 + kg * 16);
#pragma unroll
      for (int i = 0; i < IT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          cc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[j], cc[i][j], 0, 0, 0);
          cc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][i], b[j], cc[i][j], 0, 0, 0);
          cc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2][i], b[j], cc[i][j], 0, 0, 0);
        }
    }
    const int q = (ch - c0) % cps, slice = (ch - c0) / cps;  // chunk -> slice -> half total
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        sl[i][j] = q == 0 ? cc[i][j] : sl[i][j] + cc[i][j];
        if (q == cps - 1) tot[i][j] = slice == 0 ? sl[i][j] : tot[i][j] + sl[i][j];
      }
  };
  // Four register sets in a ring: while chunk ch is multiplied (LDS buffer
  // ch % 2), chunk ch + 1 is moved from registers to the other buffer and chunks
  // ch + 2 and ch + 3 are in flight, so a load has two chunks of products to
  // arrive.  Each half is a whole number of 4-chunk slices, so the loop is
  // unrolled by 4 and every ring index is a constant; past the end the last
  // chunk is fetched again (in bounds, never used) and the code stays
  // branch-free.
  Pre pr[4];
  fetch(c0, pr[0]);
  fetch(c0 + 1, pr[1]);
  fetch(c0 + 2, pr[2]);
  store(0, pr[0]);
  __syncthreads();
  for (int ch = c0; ch < c1; ch += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      fetch(min(ch + u + 3, c1 - 1), pr[(u + 3) & 3]);
      __builtin_amdgcn_sched_barrier(0);  // keep the new loads ahead of the waits for older ones
      store((u + 1) & 1, pr[(u + 1) & 3]);
      compute(u & 1, ch + u);
      __syncthreads();
    }
  }
  float* out = part + (size_t)half * T * E;
#pragma unroll
  for (int i = 0; i < IT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + we * 16 * IT + i * 16 + 4 * kg + r, t = t0 + wt * 32 + j * 16 + lr;
        if (e < E && t < T) out[(size_t)t * E + e] = tot[i][j][r];
      }
}

// ---------------------------------------------------------------------------
// Router partial logits for batches of 4096 tokens and more, larger tiles
// (bf16 x, d a multiple of 256): blocks of 128 tokens x 64 experts over one
// half of K, 4 waves of 64 tokens x 32 experts (8 products per 32-deep step
// and plane: each x fragment read from LDS feeds 2 of them, each weight
// fragment 4, against 1 and 2 in router_tile_kernel).  Per 64-deep chunk both
// operands go through LDS already in operand order (1 KB per 16 rows x 32 K):
// x gathered per token, the weights split while staged into their three exact
// bf16 planes.  Two LDS buffers, two register sets: a chunk's loads are issued
// two chunks before it is multiplied.  Sum order per logit as in
// router_tile_kernel and the K-split kernel (a chain of six products per chunk
// from zero; four chunks into a slice in order; the half's slices in order),
// so the logits are the same bit for bit.  (Weights split once at load time
// and copied instead were measured slower: their staging registers took the
// kernel past 256, to one wave per SIMD.)
// ---------------------------------------------------------------------------
template <int NJ>
__global__ __launch_bounds__(256) void router_tile2_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ W, float* __restrict__ part,
                                                           int T, int d, int E, int gsl,
                                                           int32_t* __restrict__ status) {
  constexpr int NS = 2, KC = 64, TT = 32 * NJ, TE = 64;
  constexpr int XB = (TT / 16) * NS * 1024;  // x bytes per chunk: [token tile][step][lane]
  constexpr int WB = 3 * 4 * NS * 1024;      // weight bytes per chunk: [plane][expert tile][step][lane]
  constexpr int XP = XB / 16 / 256;          // 16-byte x pieces per thread per chunk
  constexpr int WP = 4 * NS * 64 / 256;      // 8-weight slots per thread per chunk
  static_assert(XP * 16 * 256 == XB && WP >= 1, "tile shape");
  __shared__ __align__(16) uint8_t lds[2][XB + WB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, kg = lane >> 4;
  const int wt = wave & 1, we = wave >> 1;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE, half = blockIdx.z;
  if (blockIdx.x == 0 && blockIdx.y == 0 && half == 0 && tid == 0) *status = 0;
  const int c0 = half ? gsl * 4 : 0, c1 = half ? d / KC : gsl * 4;  // a multiple of 4 chunks, >= 4
  struct Set {
    v4i xv[XP];
    v4i wv[2 * WP];
  };
  auto fetch = [&](int ch, Set& S) {
    const int ks0 = ch * NS;
#pragma unroll
    for (int u = 0; u < XP; ++u) {
      const int i = tid + u * 256, tt = i / (NS * 64), ks = (i / 64) % NS, l = i % 64;
      const int t = min(t0 + 16 * tt + (l & 15), T - 1);
      S.xv[u] = *(const v4i*)(x + (size_t)t * d + 32 * (ks0 + ks) + 8 * (l >> 4));
    }
#pragma unroll
    for (int u = 0; u < WP; ++u) {
      const int sidx = tid + u * 256, et = sidx / (NS * 64), ks = (sidx / 64) % NS, l = sidx % 64;
      const int e = min(e0 + 16 * et + (l & 15), E - 1);
      const float* wp = W + (size_t)e * d + 32 * (ks0 + ks) + 8 * (l >> 4);
      S.wv[2 * u] = *(const v4i*)wp;
      S.wv[2 * u + 1] = *(const v4i*)(wp + 4);
    }
  };
  auto store = [&](int buf, const Set& S) {
    // Rows past T or E hold a clamped copy of the last row; the outputs they
    // feed are never stored.
    uint8_t* L = lds[buf];
#pragma unroll
    for (int u = 0; u < XP; ++u) *(v4i*)(L + (tid + u * 256) * 16) = S.xv[u];
#pragma unroll
    for (int u = 0; u < WP; ++u) {
      const int sidx = tid + u * 256;
      const v4i a = S.wv[2 * u], b = S.wv[2 * u + 1];
      const float w[8] = {__int_as_float(a[0]), __int_as_float(a[1]), __int_as_float(a[2]), __int_as_float(a[3]),
                          __int_as_float(b[0]), __int_as_float(b[1]), __int_as_float(b[2]), __int_as_float(b[3])};
      v8bf hi, mid, lo;
      split3_bf16(w, hi, mid, lo);
      *(v8bf*)(L + XB + (0 * 4 * NS * 64 + sidx) * 16) = hi;
      *(v8bf*)(L + XB + (1 * 4 * NS * 64 + sidx) * 16) = mid;
      *(v8bf*)(L + XB + (2 * 4 * NS * 64 + sidx) * 16) = lo;
    }
  };
  v4f tot[2][NJ], sl[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) tot[i][j] = sl[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf, int ch) {
    const uint8_t* L = lds[buf];
    v4f cc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) cc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NS; ++ks) {  // lane holds K = 32*ks + 8*kg + [0, 8)
      v8bf b[NJ], a[3][2];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[j] = *(const v8bf*)(L + ((wt * NJ + j) * NS + ks) * 1024 + 16 * lane);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[p][i] = *(const v8bf*)(L + XB + ((p * 4 + 2 * we + i) * NS + ks) * 1024 + 16 * lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          cc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[j], cc[i][j], 0, 0, 0);
          cc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][i], b[j], cc[i][j], 0, 0, 0);
          cc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2][i], b[j], cc[i][j], 0, 0, 0);
        }
    }
    const int q = (ch - c0) % 4, slice = (ch - c0) / 4;  // chunk -> slice -> half total
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        sl[i][j] = q == 0 ? cc[i][j] : sl[i][j] + cc[i][j];
        if (q == 3) tot[i][j] = slice == 0 ? sl[i][j] : tot[i][j] + sl[i][j];
      }
  };
  // Chunk c sits in register set (c - c0) % 2 from its fetch, two chunks ahead,
  // to its store into LDS buffer (c - c0) % 2; the half is an even number of
  // chunks, so the loop is unrolled by two and the sets are named statically.
  Set sa, sb;
  fetch(c0, sa);
  fetch(c0 + 1, sb);
  store(0, sa);
  fetch(c0 + 2, sa);
  __syncthreads();
  for (int ch = c0; ch < c1; ch += 2) {
    store(1, sb);  // chunk ch + 1 into the buffer chunk ch - 1 used
    if (ch + 3 < c1) fetch(ch + 3, sb);
    __builtin_amdgcn_sched_barrier(0);  // keep the new loads ahead of the waits for older ones
    compute(0, ch);
    __syncthreads();
    if (ch + 2 < c1) {
      store(0, sa);
      if (ch + 4 < c1) fetch(ch + 4, sa);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(1, ch + 1);
    __syncthreads();
  }
  float* out = part + (size_t)half * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 32 * we + 16 * i + 4 * kg + r, t = t0 + 16 * NJ * wt + 16 * j + lr;
        if (e < E && t < T) out[(size_t)t * E + e] = tot[i][j][r];
      }
}

// ---------------------------------------------------------------------------
// The router weights as three bf16 planes in matrix-core operand order, written
// once per layer by moe_pack_router: the exact split above (w = hi + mid + lo),
// so products of the planes are the products the other kernels form from the
// fp32 weights.  Fragment (expert tile et of 16, 32-deep K step ks, plane p) is
// 1 KB at 1024 * ((et * (d/32) + ks) * 3 + p); lane l's 16 bytes hold expert
// 16 et + l%16, K = 32 ks + 8 (l/16) + [0, 8).  Experts past E are zero.
// One thread per (expert tile, K step, lane).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_router_planes_kernel(const float* __restrict__ W,
                                                                 uint8_t* __restrict__ planes, int d, int E,
                                                                 int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int l = (int)(i & 63), nks = d / 32;
  const int64_t f = i >> 6;  // et * nks + ks
  const int ks = (int)(f % nks), et = (int)(f / nks);
  const int e = 16 * et + (l & 15), k = 32 * ks + 8 * (l >> 4);
  float w[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (e < E) {
    const float4 a = *(const float4*)(W + (size_t)e * d + k), b = *(const float4*)(W + (size_t)e * d + k + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  v8bf hi, mid, lo;
  split3_bf16(w, hi, mid, lo);
  uint8_t* o = planes + (size_t)f * 3 * 1024 + 16 * l;
  *(v8bf*)o = hi;
  *(v8bf*)(o + 1024) = mid;
  *(v8bf*)(o + 2048) = lo;
}

#ifndef MOE_RP_MINB
#define MOE_RP_MINB 2  // planes kernel: blocks per CU the registers must allow
#endif
// ---------------------------------------------------------------------------
// Router partial logits for long inputs from the packed planes: blocks of
// 32*NJ tokens x 64 experts over one half of K, 4 waves of 16*NJ tokens x 32
// experts.  A stage is KS 32-deep K steps; its operands are 2*NJ*KS + 12*KS
// fragments of 1 KB (x gathered per token in operand order, then per expert
// tile its K steps of the three planes, one contiguous run), which the waves
// move straight into LDS (16 bytes per lane, no registers, no conversion), NB
// stage buffers in a ring, a stage's loads issued NB - 1 stages before it is
// multiplied.  Sum order per logit as in the other router kernels (a chain of
// six products per 64-deep chunk from zero, hi, mid, lo per K step; four
// chunks into a slice in order; the half's slices in order), so the logits are
// the same bit for bit.
// ---------------------------------------------------------------------------
template <int NJ, int KS, int NB>
__global__ __launch_bounds__(256, MOE_RP_MINB) void router_planes_kernel(const uint16_t* __restrict__ x,
                                                                         const uint8_t* __restrict__ planes,
                                                                         float* __restrict__ part, int T, int d,
                                                                         int E, int gsl,
                                                                         int32_t* __restrict__ status) {
  constexpr int NXF = 2 * NJ * KS, NF = NXF + 12 * KS, FPW = NF / 4;  // fragments per stage, per wave
  constexpr int BUF = NF * 1024;
  static_assert(FPW * 4 == NF && (KS == 1 || KS == 2), "fragments per wave");
  __shared__ __align__(16) uint8_t lds[NB * BUF];
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, kg = lane >> 4, wt = wave & 1, we = wave >> 1;
  const int t0 = blockIdx.x * (32 * NJ), e0 = blockIdx.y * 64, half = blockIdx.z;
  if (blockIdx.x == 0 && blockIdx.y == 0 && half == 0 && tid == 0) *status = 0;
  const int c0 = half ? gsl * 4 : 0, c1 = half ? d / 64 : gsl * 4;  // a multiple of 4 chunks, >= 4
  const int s0 = c0 * 2 / KS, s1 = c1 * 2 / KS;                    // stages of the half
  const int nks = d / 32, n_et = (E + 15) / 16;
  // Wave w moves fragments w*FPW .. w*FPW + FPW - 1 of every stage; per
  // fragment the lane's source at stage 0 (a stage adds 64*KS bytes of x row,
  // or 3*KS KB of planes) and its LDS slot.
  const uint8_t* src[FPW];
  bool isx[FPW];
#pragma unroll
  for (int u = 0; u < FPW; ++u) {
    const int f = wave * FPW + u;
    isx[u] = f < NXF;
    if (f < NXF) {  // token tile f/KS, K step f%KS
      const int t = min(t0 + 16 * (f / KS) + lr, T - 1);
      src[u] = (const uint8_t*)(x + (size_t)t * d) + 64 * (f % KS) + 16 * kg;
    } else {  // expert tile g/(3 KS), then [K step][plane]
      const int g = f - NXF, et = min(e0 / 16 + g / (3 * KS), n_et - 1);
      src[u] = planes + ((size_t)et * nks * 3 + g % (3 * KS)) * 1024 + 16 * lane;
    }
  }
  auto issue = [&](int st) {
    uint8_t* L = lds + (st % NB) * BUF;
#pragma unroll
    for (int u = 0; u < FPW; ++u) {
      const size_t off = isx[u] ? (size_t)st * 64 * KS : (size_t)st * 3072 * KS;
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[u] + off),
                                       (__attribute__((address_space(3))) void*)(L + (wave * FPW + u) * 1024), 16, 0,
                                       0);
    }
  };
  v4f tot[2][NJ], sl[2][NJ], cc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) tot[i][j] = sl[i][j] = cc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int st) {
    const uint8_t* L = lds + (st % NB) * BUF;
    // All of the stage's fragments are requested before the first product
    // (lane holds K = 32*ks + 8*kg + [0, 8)); within a step the products run
    // plane by plane over all 2 x NJ accumulators, so consecutive products are
    // independent while each accumulator still sees hi, mid, lo per step.
    v8bf b[KS][NJ], a[KS][3][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[ks][j] = *(const v8bf*)(L + (KS * (wt * NJ + j) + ks) * 1024 + 16 * lane);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          a[ks][p][i] = *(const v8bf*)(L + (NXF + 3 * KS * (2 * we + i) + 3 * ks + p) * 1024 + 16 * lane);
    }
    __builtin_amdgcn_sched_barrier(0);  // every read in flight before the first product waits
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int kk = st * KS + ks;  // K step within the row; even steps open a 64-deep chunk
      if (kk % 2 == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) cc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            cc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks][p][i], b[ks][j], cc[i][j], 0, 0, 0);
      if (kk % 2 == 1) {
        const int q = (kk / 2 - c0) % 4, slice = (kk / 2 - c0) / 4;  // chunk -> slice -> half total
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            sl[i][j] = q == 0 ? cc[i][j] : sl[i][j] + cc[i][j];
            if (q == 3) tot[i][j] = slice == 0 ? sl[i][j] : tot[i][j] + sl[i][j];
          }
      }
    }
  };
  // vmcnt waits (expcnt and lgkmcnt left open): stage st has landed once at
  // most the loads of the stages issued after it are outstanding.
  constexpr int kWaitSteady = ((FPW * (NB - 2)) & 15) | (((FPW * (NB - 2)) >> 4) << 14) | (7 << 4) | (15 << 8);
  constexpr int kWaitAll = (7 << 4) | (15 << 8);
  static_assert(FPW * (NB - 2) < 64, "vmcnt range");
#pragma unroll
  for (int u = 0; u < NB - 1; ++u)
    if (s0 + u < s1) issue(s0 + u);
  for (int st = s0; st < s1; ++st) {
    // Wait for this wave's loads of stage st, then for every wave's (the
    // barrier), which also frees the buffer stage st - 1 was read from.
    if (st + NB - 2 < s1) __builtin_amdgcn_s_waitcnt(kWaitSteady);
    else __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (st + NB - 1 < s1) issue(st + NB - 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(st);
  }
  float* out = part + (size_t)half * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = e0 + 32 * we + 16 * i + 4 * kg + r, t = t0 + 16 * NJ * wt + 16 * j + lr;
        if (e < E && t < T) out[(size_t)t * E + e] = tot[i][j][r];
      }
}

// ---------------------------------------------------------------------------
// Router logits for fp32 activations: plain fp32 multiply-add, each logit one
// chain over the columns in order; tiles of TT tokens x TE experts, each of
// the 256 threads owning a (TT/16) x (TE/16) register tile.  The inputs go
// through LDS (transposed, padded) in chunks of 64 columns, read from memory
// with 16-byte loads two chunks ahead, so that a launch of few blocks (short
// batches) waits for about one memory round trip instead of one per chunk.
// ---------------------------------------------------------------------------
template <int TT, int TE>
__global__ __launch_bounds__(256) void router_f32_kernel(const float* __restrict__ x, const float* __restrict__ W,
                                                          float* __restrict__ logits, int T, int d, int E,
                                                          int32_t* __restrict__ status) {
  constexpr int KC = 64, MT = TT / 16, ME = TE / 16;
  constexpr int XV = TT * KC / 4 / 256, WV = TE * KC / 4 / 256;  // 16-byte loads per thread and chunk
  static_assert(XV >= 1 && WV >= 1, "every thread loads a piece of both tiles");
  __shared__ float xs[KC][TT + 1];
  __shared__ float ws[KC][TE + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int t0 = blockIdx.x * TT, e0 = blockIdx.y * TE;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *status = 0;
  // piece u of a chunk: row i / 16, columns 4 (i % 16) + [0, 4), i = tid + 256 u
  float4 xr[2][XV], wr[2][WV];
  auto load = [&](auto B, int k0) {
    constexpr int b = decltype(B)::value;
#pragma unroll
    for (int u = 0; u < XV; ++u) {
      const int i = tid + 256 * u, t = t0 + (i >> 4);
      xr[b][u] = t < T ? *(const float4*)(x + (size_t)t * d + k0 + 4 * (i & 15)) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < WV; ++u) {
      const int i = tid + 256 * u, e = e0 + (i >> 4);
      wr[b][u] = e < E ? *(const float4*)(W + (size_t)e * d + k0 + 4 * (i & 15)) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  float acc[MT][ME];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < ME; ++j) acc[i][j] = 0.f;
  const int nk = d / KC;
  // chunk kc: its registers to LDS, the loads of chunk kc + 2 issued, products
  auto step = [&](auto B, int kc) {
    constexpr int b = decltype(B)::value;
    __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
    for (int u = 0; u < XV; ++u) {
      const int i = tid + 256 * u, r = i >> 4, c = 4 * (i & 15);
      xs[c][r] = xr[b][u].x;
      xs[c + 1][r] = xr[b][u].y;
      xs[c + 2][r] = xr[b][u].z;
      xs[c + 3][r] = xr[b][u].w;
    }
#pragma unroll
    for (int u = 0; u < WV; ++u) {
      const int i = tid + 256 * u, r = i >> 4, c = 4 * (i & 15);
      ws[c][r] = wr[b][u].x;
      ws[c + 1][r] = wr[b][u].y;
      ws[c + 2][r] = wr[b][u].z;
      ws[c + 3][r] = wr[b][u].w;
    }
    __syncthreads();
    if (kc + 2 < nk) load(B, (kc + 2) * KC);
#pragma unroll 8
    for (int k = 0; k < KC; ++k) {
      float a[MT], bb[ME];
#pragma unroll
      for (int i = 0; i < MT; ++i) a[i] = xs[k][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < ME; ++j) bb[j] = ws[k][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < ME; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
  };
  load(Ic<0>{}, 0);
  if (nk > 1) load(Ic<1>{}, KC);
  int kc = 0;
  for (; kc + 1 < nk; kc += 2) {
    step(Ic<0>{}, kc);
    step(Ic<1>{}, kc + 1);
  }
  if (kc < nk) step(Ic<0>{}, kc);
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
// Top-k + weights + dispatch.  Block = 16 waves over one chunk of `tpc` tokens
// (wave w takes tokens w, w+16, ...); lane l owns the candidate experts
// e = l + 64 j of its token.
//
// Free: selection score = logit + bias ([port] part 1 of "Taking it apart":
// router score plus a per-expert selection bias); k rounds of a wave-wide
// maximum of the 64-bit key give the experts in descending score, lowest index
// on ties.  Forced ([bench] "The gate, forced"): the recorded ids, in the given
// slot order; an id outside [0, E) flags the status word, becomes -1 with
// weight 0, and the token's other slots are renormalised among themselves.
// Weights: softmax over the chosen experts' unbiased logits, normalisation sum
// in slot order.
//
// Dispatch ([port] part 3 and its update: the expert matmul consumes (token,
// expert) rows sorted by expert): a stable counting sort of the pairs
// p = t*k + j by expert.  The block's pairs get an LDS-atomic histogram
// (integer, order-free) and each pair's rank among the equal ids before it in
// the chunk.  A single block (all pairs in one chunk) finishes the sort in
// place: scan, counts, offsets, perm, inv_perm.  With several chunks the block
// writes its histogram and ranks; dispatch_scan_kernel and
// dispatch_place_kernel follow as separate launches (the launch boundary makes
// every chunk's writes visible, so no block waits on another).
// ---------------------------------------------------------------------------
constexpr int kMaxChunkPairs = 1024;

struct TopkArgs {
  const float* logits;   // [T][E]
  const float* bias;     // [E] or null
  const int32_t* forced; // [T][k] or null (free routing)
  int T, E, k, tpc;      // tpc: tokens per chunk (block)
  int32_t* idx;          // [T][k]
  float* w;              // [T][k]
  int32_t* chunk_hist;   // [n_chunks][E]
  int32_t* local_rank;   // [P]
  int32_t* counts;       // [E]
  int32_t* offsets;      // [E+1]
  int32_t* perm;         // [P]
  int32_t* inv_perm;     // [P]
  int32_t* status;
};

// One token's selection by one wave (lane l holds the candidates e = l + 64 j
// with logits lv[j]): writes idx and w of token t and returns, in lane r < k,
// the id of slot r (other lanes: -1).
template <int J, bool FORCED>
__device__ __forceinline__ int route_token(const TopkArgs& a, int t, const float (&lv)[J], int lane) {
  const int E = a.E, k = a.k;
  int sel[kMaxTopK];
  float sl[kMaxTopK];
  if (FORCED) {
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
      sel[r] = -1;
      sl[r] = 0.f;
      if (r < k) {
        const int e = a.forced[(size_t)t * k + r];
        float mine = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (lane + 64 * j == e) mine = lv[j];
        const float le = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), e & 63));
        if (e >= 0 && e < E) {
          sel[r] = e;
          sl[r] = le;
        } else {
          bad = true;
        }
      }
    }
    if (bad && lane == 0) *a.status = -5;  // MOE_ERR_FORCED_INDEX; every writer stores the same value
  } else {
    uint64_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      key[j] = e < E ? select_key(a.bias ? lv[j] + a.bias[e] : lv[j], e) : 0;
    }
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
      sel[r] = -1;
      sl[r] = 0.f;
      if (r < k) {
        // wave-wide maximum of the 64-bit key: the score word first; when one
        // lane holds it (the usual case) its index word is read directly,
        // otherwise the index words of the tied lanes are maximised too
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < J; ++j) best = key[j] > best ? key[j] : best;
        const uint32_t bhi = (uint32_t)(best >> 32);
        const uint32_t hi = wave_umax(bhi);
        const uint64_t tied = __ballot(bhi == hi);
        uint32_t lo;
        if (__popcll(tied) == 1)
          lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, __builtin_ctzll(tied));
        else
          lo = wave_umax(bhi == hi ? (uint32_t)best : 0u);
        const int e = (int)(~lo);
        float mine = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j)
          if (lane + 64 * j == e) {
            key[j] = 0;
            mine = lv[j];
          }
        sel[r] = e;
        sl[r] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), e & 63));
      }
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r)
    if (r < k && sel[r] >= 0) m = fmaxf(m, sl[r]);
  float ex[kMaxTopK], Z = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    ex[r] = 0.f;
    if (r < k && sel[r] >= 0) {
      ex[r] = expf(sl[r] - m);
      Z = Z + ex[r];
    }
  }
  int mine_id = -1;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r)
    if (r < k && lane == r) {
      a.idx[(size_t)t * k + r] = sel[r];
      a.w[(size_t)t * k + r] = sel[r] >= 0 ? ex[r] / Z : 0.f;
      mine_id = sel[r];
    }
  return mine_id;
}

// LDS of the block-wide dispatch step.
struct DispatchLds {
  int32_t hist[kMaxExperts];  // whole sort: offsets at the end
  int32_t cnt[kMaxExperts];   // whole sort: counts
  int32_t wave_cnt[16 * kMaxExperts];
  int32_t tmp[17];
};

// Dispatch step over the up-to-1024 pairs of one block (1024 threads; thread
// tid holds pair p with id e, or e = -1 for none/invalid).  Rank of a pair
// among the equal ids before it: within its wave from ballots (lanes whose id
// agrees on every bit), plus the same id's count in earlier waves (per-wave
// counts scanned in wave order).  `whole`: the block holds every pair, so the
// counting sort is finished here (counts, offsets, perm, inv_perm); otherwise
// the block's histogram and ranks go to chunk_hist / local_rank.
__device__ __forceinline__ int dispatch_block(const TopkArgs& a, DispatchLds& s, int e, int p, bool live,
                                              bool whole, int n_pairs) {
  const int nw = (n_pairs + 63) / 64;  // waves that hold pairs (threads past n_pairs have e = -1)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  uint64_t peers = __ballot(1);
#pragma unroll
  for (int bit = 0; bit < 10; ++bit) {  // ids are -1 .. kMaxExperts-1 < 2^10 (as 10-bit two's complement)
    const uint64_t b = __ballot((e >> bit) & 1);
    peers &= ((e >> bit) & 1) ? b : ~b;
  }
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  const int in_wave = __popcll(peers & below);
  const bool leader = (peers & below) == 0;  // lowest lane of its id group
  for (int i = tid; i < nw * E; i += 1024) s.wave_cnt[i] = 0;
  __syncthreads();
  if (leader && e >= 0) s.wave_cnt[wave * E + e] = __popcll(peers);
  __syncthreads();
  for (int i = tid; i < E; i += 1024) {  // exclusive scan over waves, in wave order; totals -> hist
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = s.wave_cnt[w * E + i];
      s.wave_cnt[w * E + i] = run;
      run += c;
    }
    s.hist[i] = run;
  }
  __syncthreads();
  const int rank = e >= 0 ? s.wave_cnt[wave * E + e] + in_wave : 0;
  if (!whole) {
    if (live) a.local_rank[p] = rank;
    for (int i = tid; i < E; i += 1024) a.chunk_hist[(size_t)blockIdx.x * E + i] = s.hist[i];
    return -1;
  }
  const int cnt = tid < E ? s.hist[tid] : 0;
  int total;
  const int off = block1024_excl_scan(cnt, s.tmp, &total);
  if (tid < E) {
    a.counts[tid] = cnt;
    a.offsets[tid] = off;
    s.hist[tid] = off;
    s.cnt[tid] = cnt;
  }
  if (tid == 0) a.offsets[E] = total;
  __syncthreads();
  int q = -1;
  if (live) {
    if (e >= 0) {
      q = s.hist[e] + rank;
      a.perm[q] = p;
      a.inv_perm[p] = q;
    } else {
      a.inv_perm[p] = -1;
    }
    if (p >= total) a.perm[p] = -1;
  }
  return q;
}

// Logits of token t for the candidates e = lane + 64 j.  The router left n_parts
// partial sums per logit, in K order; the logit is (parts [0, gs) added in
// order) + (parts [gs, n_parts) added in order): the K-split router writes one
// part per 256-deep slice (gs = half of them), the tiled router one part per
// half of K (gs = 1), so both give the same sum bit for bit.  Written to
// logits_out when given.  The parts are requested QB at a time (all J
// candidates at once), then added: QB = 8 after the K-split router, 2 after the
// tiled one (at most two parts; a larger batch would issue loads for parts
// that do not exist, masked off but still issued).
template <int J, int QB>
__device__ __forceinline__ void gather_logits(const float* __restrict__ part, int n_parts, int gs, int T, int E,
                                              int t, int lane, float* __restrict__ logits_out, float (&lv)[J]) {
  float h0[J], h1[J];
#pragma unroll
  for (int j = 0; j < J; ++j) h0[j] = h1[j] = 0.f;
  for (int q0 = 0; q0 < n_parts; q0 += QB) {
    float v[QB][J];
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        v[q][j] = (q0 + q < n_parts && e < E) ? part[((size_t)(q0 + q) * T + t) * E + e] : 0.f;
      }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int qq = q0 + q;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (qq < gs) h0[j] = qq == 0 ? v[q][j] : h0[j] + v[q][j];
        else if (qq < n_parts) h1[j] = qq == gs ? v[q][j] : h1[j] + v[q][j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) lv[j] = gs < n_parts ? h0[j] + h1[j] : h0[j];
  if (logits_out) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      if (e < E) logits_out[(size_t)t * E + e] = lv[j];
    }
  }
}

// Top-k + dispatch over chunks of `tpc` tokens (long inputs): block = 16 waves,
// wave w takes tokens w, w+16, ... of its chunk.
template <int J, bool FORCED>
__global__ __launch_bounds__(1024) void topk_dispatch_kernel(TopkArgs a, const float* __restrict__ part, int n_parts,
                                                            int gs, float* __restrict__ logits_out) {
  __shared__ DispatchLds s;
  __shared__ int32_t ids[kMaxChunkPairs];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, k = a.k, T = a.T;
  const int tok0 = blockIdx.x * a.tpc;

  for (int tl = wave; tl < a.tpc; tl += 16) {
    const int t = tok0 + tl;
    if (t >= T) {
      if (lane < k) ids[tl * k + lane] = -1;
      continue;
    }
    float lv[J];
    gather_logits<J, 2>(part, n_parts, gs, T, E, t, lane, logits_out, lv);
    const int id = route_token<J, FORCED>(a, t, lv, lane);
    if (lane < k) ids[tl * k + lane] = id;
  }
  __syncthreads();
  const int np = a.tpc * k, p = blockIdx.x * np + tid;
  const bool live = tid < np && p < T * k;
  dispatch_block(a, s, tid < np ? ids[tid] : -1, p, live, gridDim.x == 1, np);
}

// Short inputs, step 2: one wave per token.  The router left n_parts partial
// dot products per logit (K slices); they are added in slice order, the sum is
// the logit (written to logits_out when given), then the selection.
template <int J, bool FORCED>
__global__ __launch_bounds__(64) void topk_small_kernel(TopkArgs a, const float* __restrict__ part, int n_parts,
                                                        int gs, float* __restrict__ logits_out) {
  const int t = blockIdx.x, lane = threadIdx.x;
  const int E = a.E, T = a.T;
  float lv[J];
  gather_logits<J, 8>(part, n_parts, gs, T, E, t, lane, logits_out, lv);
  route_token<J, FORCED>(a, t, lv, lane);
}

// Short inputs, step 3: block 0 does the whole counting sort (T * k <= 1024)
// and then the dispatch plan (per-row info, block schedules, see moe_plan.h);
// the other blocks quantise the activations (FP8 weights), 16 chunks of 512
// elements each (one per wave).
__global__ __launch_bounds__(1024) void dispatch_small_kernel(TopkArgs a, PlanCtx pc) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (blockIdx.x > 0) {
    const int cpr = (pc.gpr + 3) / 4, u = (blockIdx.x - 1) * 16 + (tid >> 6);  // one 512-element chunk per wave
    if (u < pc.n_rows * cpr) quantize_groups4<true>(pc.x, u / cpr, 4 * (u % cpr), pc.gpr, pc.xq, pc.sx, lane);
    return;
  }
  __shared__ DispatchLds s;
  __shared__ PlanLds pl;
  const int T = a.T, P = T * a.k, p = tid;
  const bool live = p < P;
  const int e = live ? a.idx[p] : -1;
  const float wp = a.w[live ? p : 0];  // requested with the ids: one round trip for both
  const int q = dispatch_block(a, s, e, p, live, true, P);
  if (q >= 0) {
    pc.ri.tok[q] = p / a.k;
    pc.ri.prow[q] = p;
    pc.ri.w[q] = wp;
  }
  if (pc.pa.has_shared)
    for (int t = tid; t < T; t += 1024) {
      pc.ri.tok[P + t] = t;
      pc.ri.prow[P + t] = P + t;
      pc.ri.w[P + t] = 1.f;
    }
  PlanArgs pa = pc.pa;
  pa.counts = s.cnt;
  pa.offsets = s.hist;
  const int total = plan_tables<1024>(pa, pl);
  plan_scatter<1024>(pa, pl, total);
}

// Several chunks, step 3: one block per expert e scans e's chunk histogram
// entries in chunk order, in place (entry [c][e] becomes the pairs of e in
// chunks before c), and writes counts[e].  Each thread takes a run of chunks.
__global__ __launch_bounds__(256) void dispatch_scan_kernel(int32_t* __restrict__ chunk_hist, int n_chunks, int E,
                                                             int32_t* __restrict__ counts) {
  __shared__ int32_t tmp[17];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int per = (n_chunks + 255) / 256, c0 = min(tid * per, n_chunks), c1 = min(c0 + per, n_chunks);
  int sum = 0;
  for (int c = c0; c < c1; ++c) sum += chunk_hist[(size_t)c * E + e];
  int total;
  int run = block_excl_scan<256>(sum, tmp, &total);
  for (int c = c0; c < c1; ++c) {
    int32_t* h = chunk_hist + (size_t)c * E + e;
    const int v = *h;
    *h = run;
    run += v;
  }
  if (tid == 0) counts[e] = total;
}

// Exclusive scan of counts[0..E) into offs[0..E] (LDS) by a 256-thread block.
__device__ __forceinline__ void block_offsets(const int32_t* __restrict__ counts, int E, int32_t* offs,
                                              int32_t* tmp) {
  constexpr int PER = (kMaxExperts + 255) / 256;
  int v[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = PER * threadIdx.x + i;
    v[i] = e < E ? counts[e] : 0;
    sum += v[i];
  }
  int total;
  int run = block_excl_scan<256>(sum, tmp, &total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = PER * threadIdx.x + i;
    if (e < E) offs[e] = run;
    run += v[i];
  }
  if (threadIdx.x == 0) offs[E] = total;
  __syncthreads();
}

// Long inputs, step 4, one launch: placement of every pair, q = offsets[e] +
// (pairs of e in earlier chunks) + rank in the chunk, with the per-row info of
// the placed pairs (blocks [0, npl); each derives the expert offsets from the
// counts, block 0 also stores them); the shared expert's rows (next nsr
// blocks); the block schedules (next npb blocks, kPlanEntries entries each);
// the activation quantisation (the rest, one row per wave).
constexpr int kPlanEntries = 512;

__global__ __launch_bounds__(256) void dispatch_place_kernel(const int32_t* __restrict__ idx, int P, int E, int np,
                                                              const int32_t* __restrict__ chunk_prefix,
                                                              const int32_t* __restrict__ local_rank,
                                                              const int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm,
                                                              int32_t* __restrict__ inv_perm,
                                                              const float* __restrict__ topk_w, PlanCtx pc,
                                                              int npl, int nsr, int npb) {
  const int tid = threadIdx.x, blk = blockIdx.x;
  __shared__ int32_t offs[kMaxExperts + 1], tmp[17];
  if (blk < npl) {
    const int p = min(blk * 256 + tid, P - 1);
    const int e = idx[p];
    const int cp = (e >= 0 && e < E) ? chunk_prefix[(size_t)(p / np) * E + e] + local_rank[p] : 0;
    block_offsets(counts, E, offs, tmp);
    if (blk == 0)
      for (int i = tid; i <= E; i += 256) offsets[i] = offs[i];
    if (blk * 256 + tid >= P) return;
    if (e >= 0 && e < E) {
      const int q = offs[e] + cp;
      perm[q] = p;
      inv_perm[p] = q;
      pc.ri.tok[q] = p / pc.k;
      pc.ri.prow[q] = p;
      pc.ri.w[q] = topk_w[p];
    } else {
      inv_perm[p] = -1;
    }
    if (p >= offs[E]) perm[p] = -1;
    return;
  }
  if (blk < npl + nsr) {
    const int t = (blk - npl) * 256 + tid;
    if (t < pc.pa.T) {
      pc.ri.tok[P + t] = t;
      pc.ri.prow[P + t] = P + t;
      pc.ri.w[P + t] = 1.f;
    }
    return;
  }
  if (blk < npl + nsr + npb) {
    __shared__ PlanLds pl;
    block_offsets(counts, E, offs, tmp);
    PlanArgs pa = pc.pa;
    pa.offsets = offs;
    const int total = plan_tables<256>(pa, pl);
    const int e0 = (blk - npl - nsr) * kPlanEntries, ne = plan_n_entries(pc.pa);
    for (int i = tid; i < kPlanEntries && e0 + i < ne; i += 256) plan_any_entry(pa, pl, total, e0 + i);
    return;
  }
  const int row = (blk - npl - nsr - npb) * 4 + (tid >> 6);
  if (row < pc.n_rows) quantize_row<true>(pc.x, row, pc.gpr, pc.xq, pc.sx, tid & 63);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Tokens per top-k block: all of them when their pairs fit one block, else 16
// (one token per wave; the per-expert scan of the chunk histograms is parallel),
// doubled while the blocks would outnumber the chip's 256 CUs and a chunk's
// pairs still fit one block: the kernel holds one 16-wave block per CU, and a
// second round of blocks costs more than a second token per wave.
constexpr int kNumCUs = 256;
int tokens_per_chunk(int T, int k) {
  if (T * k <= kMaxChunkPairs) return T > 0 ? T : 1;
  int tpc = 16;
  while ((T + tpc - 1) / tpc > kNumCUs && 2 * tpc * k <= kMaxChunkPairs) tpc *= 2;
  return tpc;
}

size_t dispatch_chunk_hist_ints(int T, int k, int E) {
  const int tpc = tokens_per_chunk(T, k);
  const int n_chunks = (T + tpc - 1) / tpc;
  return n_chunks > 1 ? (size_t)n_chunks * E : 0;
}

int router_kslice(int d) { return d % 256 == 0 ? 256 : 128; }

#ifndef MOE_SPLIT_ROUTER_MAX_T
#define MOE_SPLIT_ROUTER_MAX_T 384
#endif
// Batches of up to this many tokens use the K-split router whatever their
// dispatch path: the tiled routers' blocks (64 or more tokens x 64 experts x
// half of K) would leave most of the chip idle (measured with packed planes:
// routing 35 -> 30 us at 256 tokens; 36 -> 37 at 512 and 38 -> 48 at 1024,
// where the split's repeated weight reads cost more).
constexpr int kSplitRouterMaxT = MOE_SPLIT_ROUTER_MAX_T;

static bool split_router(int T, int k) { return (int64_t)T * k <= kMaxChunkPairs || T <= kSplitRouterMaxT; }

size_t router_part_floats(int T, int k, int d, int E, bool x_bf16) {
  if (!x_bf16) return 0;
  if (!split_router(T, k)) return (size_t)2 * T * E;  // two halves of K
  return (size_t)(d / router_kslice(d)) * T * E;
}

static TopkArgs topk_args(const RouteLaunch& L, int tpc) {
  TopkArgs a;
  a.logits = L.logits;
  a.bias = L.forced ? nullptr : L.bias;
  a.forced = L.forced;
  a.T = L.T;
  a.E = L.E;
  a.k = L.k;
  a.tpc = tpc;
  a.idx = L.idx;
  a.w = L.w;
  a.chunk_hist = L.chunk_hist;
  a.local_rank = L.local_rank;
  a.counts = L.counts;
  a.offsets = L.offsets;
  a.perm = L.perm;
  a.inv_perm = L.inv_perm;
  a.status = L.status;
  return a;
}

#define MOE_J_SWITCH(J, CASE)                                                            \
  switch (J) {                                                                           \
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)                      \
    default: return hipErrorInvalidValue;                                                \
  }

#ifndef MOE_RP_NJ_LONG
#define MOE_RP_NJ_LONG 4   // planes kernel: 16-token tiles per wave, batches of kPlanesLongT tokens and more
#endif
#ifndef MOE_RP_NB_LONG
#define MOE_RP_NB_LONG 2   // planes kernel: LDS buffers in the ring
#endif
#ifndef MOE_RP_KS_LONG
#define MOE_RP_KS_LONG 1   // planes kernel: 32-deep K steps per LDS stage (2: 4% slower at T = 8192)
#endif
#ifndef MOE_RP_KS_SHORT
#define MOE_RP_KS_SHORT 2
#endif
#ifndef MOE_RP_NJ_SHORT
#define MOE_RP_NJ_SHORT 2
#endif
#ifndef MOE_RP_NB_SHORT
#define MOE_RP_NB_SHORT 2
#endif
constexpr int kPlanesLongT = 4096;

size_t router_planes_bytes(int d, int E) { return (size_t)((E + 15) / 16) * (d / 32) * 3 * 1024; }

hipError_t launch_pack_router(const float* W, void* planes, int d, int E, hipStream_t st) {
  const int64_t n = (int64_t)((E + 15) / 16) * (d / 32) * 64;
  pack_router_planes_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(W, (uint8_t*)planes, d, E, n);
  return hipGetLastError();
}

// Router launch: bf16 activations go through the K-split kernel (short inputs)
// or the tiled kernel (long inputs), which leave partial sums that top-k adds in
// one order, so a token's logits never depend on T; fp32 activations (small
// layers) get plain logits.
static hipError_t launch_router(const RouteLaunch& L, hipStream_t st, const float*& part, int& n_parts, int& gs,
                                float*& logits_out) {
  const bool shortin = (int64_t)L.T * L.k <= kMaxChunkPairs;
  if (L.x_bf16 && !split_router(L.T, L.k)) {  // tiles over two halves of K
    const int ksl = router_kslice(L.d), ns = L.d / ksl, halves = ns > 1 ? 2 : 1;
    const dim3 grid((L.T + 63) / 64, (L.E + 63) / 64, halves);
    const uint16_t* x = (const uint16_t*)L.x;
    if (L.planes && ksl == 256 && halves == 2) {  // packed planes
      const int gsl = (ns + 1) / 2;
      if (L.T >= kPlanesLongT) {
        const dim3 g((L.T + 32 * MOE_RP_NJ_LONG - 1) / (32 * MOE_RP_NJ_LONG), (L.E + 63) / 64, 2);
        router_planes_kernel<MOE_RP_NJ_LONG, MOE_RP_KS_LONG, MOE_RP_NB_LONG><<<g, 256, 0, st>>>(
            x, L.planes, L.rpart, L.T, L.d, L.E, gsl, L.status);
      } else {
        const dim3 g((L.T + 32 * MOE_RP_NJ_SHORT - 1) / (32 * MOE_RP_NJ_SHORT), (L.E + 63) / 64, 2);
        router_planes_kernel<MOE_RP_NJ_SHORT, MOE_RP_KS_SHORT, MOE_RP_NB_SHORT><<<g, 256, 0, st>>>(
            x, L.planes, L.rpart, L.T, L.d, L.E, gsl, L.status);
      }
    } else if (ksl == 256 && halves == 2 && L.T >= 4096) {  // 128-token blocks once they fill the chip
      const dim3 g2((L.T + 127) / 128, (L.E + 63) / 64, 2);
      router_tile2_kernel<4><<<g2, 256, 0, st>>>(x, L.w_router, L.rpart, L.T, L.d, L.E, (ns + 1) / 2, L.status);
    } else if (ksl == 256)
      router_tile_kernel<2, 8><<<grid, 512, 0, st>>>((const uint16_t*)L.x, L.w_router, L.rpart, L.T, L.d, L.E,
                                                     (ns + 1) / 2, L.status);
    else
      router_tile_kernel<1, 4><<<grid, 256, 0, st>>>((const uint16_t*)L.x, L.w_router, L.rpart, L.T, L.d, L.E,
                                                     (ns + 1) / 2, L.status);
    part = L.rpart;
    n_parts = halves;
    gs = 1;
    logits_out = L.logits;
  } else if (L.x_bf16) {
    const int ksl = router_kslice(L.d), NS = ksl / 128;
    const int NC = !shortin ? 4 : (L.T <= 16 ? 1 : (L.T <= 32 ? 2 : (L.T <= 48 ? 3 : 4)));
    const dim3 grid((L.E + 15) / 16, L.d / ksl, (L.T + 16 * NC - 1) / (16 * NC));
    const uint16_t* x = (const uint16_t*)L.x;
#define MOE_SPLIT(nc, ns) \
  router_split_kernel<nc, ns><<<grid, 256, 0, st>>>(x, L.w_router, L.rpart, L.T, L.d, L.E, L.status)
    if (NS == 2) {
      if (NC == 1) MOE_SPLIT(1, 2); else if (NC == 2) MOE_SPLIT(2, 2); else if (NC == 3) MOE_SPLIT(3, 2); else MOE_SPLIT(4, 2);
    } else {
      if (NC == 1) MOE_SPLIT(1, 1); else if (NC == 2) MOE_SPLIT(2, 1); else if (NC == 3) MOE_SPLIT(3, 1); else MOE_SPLIT(4, 1);
    }
#undef MOE_SPLIT
    part = L.rpart;
    n_parts = L.d / ksl;
    gs = (n_parts + 1) / 2;
    logits_out = L.logits;
  } else {
    if (shortin) {
      const dim3 grid((L.T + 31) / 32, (L.E + 15) / 16);
      router_f32_kernel<32, 16><<<grid, 256, 0, st>>>((const float*)L.x, L.w_router, L.logits, L.T, L.d, L.E, L.status);
    } else {
      const dim3 grid((L.T + 63) / 64, (L.E + 63) / 64);
      router_f32_kernel<64, 64><<<grid, 256, 0, st>>>((const float*)L.x, L.w_router, L.logits, L.T, L.d, L.E, L.status);
    }
    part = L.logits;
    n_parts = 1;
    gs = 1;
    logits_out = nullptr;
  }
  return hipGetLastError();
}

hipError_t launch_route(const RouteLaunch& L, hipStream_t st) {
  const float* part;
  int n_parts, gs;
  float* logits_out;
  hipError_t e = launch_router(L, st, part, n_parts, gs, logits_out);
  if (e != hipSuccess) return e;
  if ((int64_t)L.T * L.k <= kMaxChunkPairs) {  // one wave per token, then a one-block dispatch
    const TopkArgs a = topk_args(L, L.T);
#define MOE_TOPK_SMALL(n)                                                                        \
  case n:                                                                                        \
    if (L.forced) topk_small_kernel<n, true><<<L.T, 64, 0, st>>>(a, part, n_parts, gs, logits_out);  \
    else topk_small_kernel<n, false><<<L.T, 64, 0, st>>>(a, part, n_parts, gs, logits_out);          \
    break;
    MOE_J_SWITCH((L.E + 63) / 64, MOE_TOPK_SMALL)
#undef MOE_TOPK_SMALL
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nqb = (L.plan.n_rows * ((L.plan.gpr + 3) / 4) + 15) / 16;
    dispatch_small_kernel<<<1 + nqb, 1024, 0, st>>>(a, L.plan);
    return hipGetLastError();
  }
  const int P = L.T * L.k;
  const int tpc = tokens_per_chunk(L.T, L.k);
  const int n_chunks = (L.T + tpc - 1) / tpc;
  const TopkArgs a = topk_args(L, tpc);
#define MOE_TOPK_CASE(n)                                                                                        \
  case n:                                                                                                       \
    if (L.forced) topk_dispatch_kernel<n, true><<<n_chunks, 1024, 0, st>>>(a, part, n_parts, gs, logits_out);        \
    else topk_dispatch_kernel<n, false><<<n_chunks, 1024, 0, st>>>(a, part, n_parts, gs, logits_out);                \
    break;
  MOE_J_SWITCH((L.E + 63) / 64, MOE_TOPK_CASE)
#undef MOE_TOPK_CASE
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  dispatch_scan_kernel<<<L.E, 256, 0, st>>>(L.chunk_hist, n_chunks, L.E, L.counts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int npl = (P + 255) / 256, nsr = L.plan.pa.has_shared ? (L.T + 255) / 256 : 0;
  const int npb = (plan_n_entries(L.plan.pa) + kPlanEntries - 1) / kPlanEntries;
  const int nqb = (L.plan.n_rows + 3) / 4;
  dispatch_place_kernel<<<(unsigned)(npl + nsr + npb + nqb), 256, 0, st>>>(
      L.idx, P, L.E, tpc * L.k, L.chunk_hist, L.local_rank, L.counts, L.offsets, L.perm, L.inv_perm, L.w, L.plan, npl, nsr,
      npb);
  return hipGetLastError();
}
#undef MOE_J_SWITCH

}  // namespace moe
