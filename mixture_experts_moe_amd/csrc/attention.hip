// The attention ops next to the mixture-of-experts layer: rotary position
// encoding, and causal attention over a sliding window or the whole context.
//
// Pages cited by title and section:
//   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
//   [bench] "We Stopped the Kolibri Benchmark Before Scoring One Answer"
//
// [port] "The gate": forty layers attend over a 513-token sliding window with
// rotary position encoding (RoPE), every fifth over the whole context with no
// positional encoding (also [bench] "The pilot that ran out of buffers, not
// memory").  [port] "Taking it apart", part 2: RoPE rotates each pair of a
// query's or key's dimensions by the position times 1/theta^(2j/D).
//
// Attention is flash-style, one pass over the keys with an online softmax, on
// the bf16 matrix cores (16x16x32).  A block holds 64 rows -- (query, head)
// pairs of one key/value head group -- in four waves of 16.  Key and value
// tiles of 64 keys go through LDS (values transposed), the next tile's loads
// in flight while the current one is computed.  The score tile is computed
// transposed, S^T = K Q^T, so that every value a lane holds belongs to the
// same row (query, head): the row's running maximum and sum sit in the four
// lanes of its column, and rescaling the output is a per-lane multiply.  The
// output is accumulated transposed as well, O^T = V^T P^T, where each lane's
// eight probabilities of a 32-key step are exactly the eight key slots the
// matrix core expects from it (keys 32c + 4(l/16) + [0,4) and + 16); they
// enter as a bf16 high part and a bf16 low part, two products, so that the
// result carries about 16 bits of each probability.
// Short query batches (decode) split the key range over blocks; a combine
// launch merges the partial (max, sum, output) triples.
#include <math.h>

#include "moe_attn.h"
#include "moe_device.h"

namespace moe {

constexpr int kAttD = 128;    // head dimension
constexpr int kAttKT = 64;    // keys per tile
constexpr int kAttRows = 64;  // (query, head) rows per block of 4 waves (8 waves: 128)
constexpr int kKStride = kAttD + 16;  // bf16 elements per LDS key row (288 bytes: 32 modulo 64)
constexpr int kVStride = kAttKT + 4;  // bf16 elements per LDS value-transposed row
constexpr int kAttSplitMax = 512;     // key splits per row (decode)

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* part_o;   // [split][Tq*Hq][D] unnormalised outputs (split launches)
  float* part_ml;  // [split][Tq*Hq][2] running max (log2 units) and sum
  int Tq, Tk, Hq, Hkv, G, qpb, q_pos0, window, n_split, tps;
  float scale_log2;  // log2(e) / sqrt(D)
};

typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

// Two floats as packed bf16 (round to nearest even, the packed conversion).
__device__ __forceinline__ uint32_t bf16x2(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t){x0, x1}, v2bf_t));
}
// Two floats as packed bf16 high parts and packed bf16 of what remains.
__device__ __forceinline__ void bf16x2_hi_lo(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const v2f_t w = {x0, x1};
  const v2bf_t h = __builtin_convertvector(w, v2bf_t);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(w - __builtin_convertvector(h, v2f_t), v2bf_t));
}

// double -> bf16, round to nearest, ties to even, exact for results in the
// normal range (the rest goes through float).
__device__ __forceinline__ uint16_t bf16_from_double(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t sign = u >> 63;
  uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  if (mag == 0) return (uint16_t)(sign << 15);
  const int e = (int)(mag >> 52) - 1023;
  if (e < -126 || e > 127) return f32_to_bf16((float)v);
  mag += 0x00000FFFFFFFFFFFull + ((mag >> 45) & 1);  // round at the 7th mantissa bit
  mag >>= 45;
  const int e2 = (int)(mag >> 7) - 1023;
  if (e2 > 127) return (uint16_t)((sign << 15) | 0x7F80);
  return (uint16_t)((sign << 15) | ((uint64_t)(e2 + 127) << 7) | (mag & 0x7F));
}

// RoPE, one block per token.  The angles (pos0 + t) * theta^(-2j/D) are formed
// and reduced modulo 2 pi in double (positions reach 10^5 radians, far beyond
// fp32's resolution), their cos and sin taken in fp32 once per token into LDS;
// then the block rotates every head's pairs (j, j + D/2) in fp32 (about 2^-22
// relative, against the bf16 result's 2^-8 rounding step), rounded once to bf16.
// V pairs per thread step: 4 (8-byte loads and stores) when D/2 is a multiple
// of 4 and x is 8-byte aligned, else 1.
template <int V>
__global__ __launch_bounds__(256) void rope_kernel(uint16_t* __restrict__ x, int H, int D, int pos0,
                                                   double log2_theta) {
  __shared__ float cs[512], sn[512];
  const int half = D / 2, t = blockIdx.x, tid = threadIdx.x;
  const double inv_two_pi = 0.15915494309189535, two_pi = 6.283185307179586;
  for (int j = tid; j < half; j += 256) {
    const double ang = (double)(pos0 + t) * exp2(-2.0 * j / D * log2_theta);
    sincosf((float)(ang - two_pi * rint(ang * inv_two_pi)), &sn[j], &cs[j]);
  }
  __syncthreads();
  uint16_t* row0 = x + (size_t)t * H * D;
  const int hv = half / V;
  for (int i = tid; i < H * hv; i += 256) {
    const int h = i / hv, j0 = (i - h * hv) * V;
    uint16_t* p = row0 + h * D;
    uint16_t lo[V], hi[V];
    if constexpr (V == 4) {
      *(uint2*)lo = *(const uint2*)(p + j0);
      *(uint2*)hi = *(const uint2*)(p + j0 + half);
    } else {
      lo[0] = p[j0];
      hi[0] = p[j0 + half];
    }
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int j = j0 + u;
      const float a = bf16_to_f32(lo[u]), b = bf16_to_f32(hi[u]);
      lo[u] = f32_to_bf16(a * cs[j] - b * sn[j]);
      hi[u] = f32_to_bf16(a * sn[j] + b * cs[j]);
    }
    if constexpr (V == 4) {
      *(uint2*)(p + j0) = *(const uint2*)lo;
      *(uint2*)(p + j0 + half) = *(const uint2*)hi;
    } else {
      p[j0] = lo[0];
      p[j0 + half] = hi[0];
    }
  }
}

// One block: NW*16 (query, head) rows of key/value head blockIdx.y, over tile
// range split blockIdx.z of the block's keys.  NW = 8 for long query batches
// (each staged tile serves 128 rows), 4 for short ones.  KS key groups of NW
// waves each: group g takes the tiles g, g + KS, ... of the range (its own LDS
// buffers, the same per-tile code), and at the end the groups' running
// (max, sum, output) states of each row are merged through LDS in group order,
// so a long batch, whose rows alone give two waves per SIMD, gets KS times
// as many waves to hide each tile's dependent chain.
template <int NW, int KS>
__global__ __launch_bounds__(NW * KS * 64) void attention_kernel(AttnArgs a) {
  constexpr int NT = NW * 64, CPT = 1024 / NT;  // threads per group; 16-byte chunks of K (and of V) per thread
  constexpr int kGroupLds = kAttKT * kKStride + kAttD * kVStride;  // bf16 elements: a K tile, a V^T tile
  __shared__ __align__(16) uint16_t lds[KS * kGroupLds];
  const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / NT);
  uint16_t* const ks = lds + grp * kGroupLds;
  uint16_t* const vts = ks + kAttKT * kKStride;
  const int tid = threadIdx.x % NT, wave = tid >> 6, lane = tid & 63, lr = lane & 15, q4 = lane >> 4;
  const int kvh = blockIdx.y;
  const int qb0 = blockIdx.x * a.qpb;  // first query of the block
  // this lane's row as the B operand of S^T (and the row whose state it keeps)
  const int row = wave * 16 + lr;
  const int qi = qb0 + row / a.G, head = kvh * a.G + row % a.G;
  const bool live = qi < a.Tq;
  const int p = a.q_pos0 + qi;  // the row's position
  // the block's key range: causal, and the window of its first query
  const int last_q = min(qb0 + a.qpb, a.Tq) - 1;
  const int k_lo = a.window > 0 ? max(0, a.q_pos0 + qb0 - a.window + 1) : 0;
  const int k_hi = a.q_pos0 + last_q + 1;
  const int n_tiles = (k_hi - k_lo + kAttKT - 1) / kAttKT;
  const int t_begin = blockIdx.z * a.tps, t_end = min(n_tiles, t_begin + a.tps);

  // the row's query, as four 8-element chunks per lane (d = 32 s + 8 q4 + [0, 8))
  v4i qr[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qr[s] = v4i{0, 0, 0, 0};
    if (live) qr[s] = *(const v4i*)(a.q + ((size_t)qi * a.Hq + head) * kAttD + 32 * s + 8 * q4);
  }

  // tile staging: 64 keys x 128 d of K and of V in 1024 16-byte chunks each,
  // CPT of each per thread.  K: chunk c is key c/16, 16-byte chunk c%16 of its
  // row.  V: the thread takes chunk ch = c/64 of two neighbouring keys,
  // 2 (c%32) and 2 (c%32) + 1 with c over the 512 pair slots, so that each
  // 4-byte LDS store of the transposed tile holds one d of both keys.
  // Each thread's chunks sit at fixed offsets from the tile's first key: the
  // key within the tile and the 16-byte column are set once, a tile adds a
  // block-uniform offset, and keys past the range are simply not loaded.
  // With two key groups (four waves per SIMD, 128 registers) the clamped,
  // unconditional loads of the first form measured faster (whole-context
  // chunk 122-126 us against 132); with one group the precomputed,
  // conditional loads (window chunk 25 against 28-31 us, decode 20.5 against
  // 22.1).
  v4i kreg[CPT], vreg[CPT];
  int kkey[CPT], vkey[CPT];
  const uint16_t *kp[CPT], *vp[CPT];
  const size_t key_stride = (size_t)a.Hkv * kAttD;  // elements from one key to the next
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int c = tid + u * NT;
    kkey[u] = c >> 4;
    kp[u] = a.k + ((size_t)kkey[u] * a.Hkv + kvh) * kAttD + (c & 15) * 8;
    const int pc = tid + (u >> 1) * NT;  // pair slot
    vkey[u] = 2 * (pc & 31) + (u & 1);
    vp[u] = a.v + ((size_t)vkey[u] * a.Hkv + kvh) * kAttD + (pc >> 5) * 8;
  }
  auto fetch = [&](int tile) {
    const int k0 = k_lo + tile * kAttKT;
    if constexpr (KS > 1) {
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int c = tid + u * NT;
        const int kk = k0 + (c >> 4);
        const size_t ko = ((size_t)min(kk, a.Tk - 1) * a.Hkv + kvh) * kAttD + (c & 15) * 8;
        kreg[u] = kk < k_hi ? *(const v4i*)(a.k + ko) : v4i{0, 0, 0, 0};
        const int pc = tid + (u >> 1) * NT;  // pair slot
        const int kv = k0 + 2 * (pc & 31) + (u & 1);
        const size_t vo = ((size_t)min(kv, a.Tk - 1) * a.Hkv + kvh) * kAttD + (pc >> 5) * 8;
        vreg[u] = kv < k_hi ? *(const v4i*)(a.v + vo) : v4i{0, 0, 0, 0};
      }
    } else {
      const size_t off = (size_t)k0 * key_stride;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        kreg[u] = v4i{0, 0, 0, 0};
        if (k0 + kkey[u] < k_hi) kreg[u] = *(const v4i*)(kp[u] + off);
        vreg[u] = v4i{0, 0, 0, 0};
        if (k0 + vkey[u] < k_hi) vreg[u] = *(const v4i*)(vp[u] + off);
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int c = tid + u * NT;
      *(v4i*)(ks + (c >> 4) * kKStride + (c & 15) * 8) = kreg[u];
    }
#pragma unroll
    for (int h = 0; h < CPT / 2; ++h) {
      const int pc = tid + h * NT;
      const uint32_t* e0 = (const uint32_t*)&vreg[2 * h];      // key 2 (pc % 32), 8 d values
      const uint32_t* e1 = (const uint32_t*)&vreg[2 * h + 1];  // the next key, same d values
      uint32_t* dst = (uint32_t*)(vts + ((pc >> 5) * 8) * kVStride + 2 * (pc & 31));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[(2 * i) * (kVStride / 2)] = (e0[i] & 0xFFFFu) | (e1[i] << 16);
        dst[(2 * i + 1) * (kVStride / 2)] = (e0[i] >> 16) | (e1[i] & 0xFFFF0000u);
      }
    }
  };

  v4f acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
  float mrow = -INFINITY, lrow = 0.f;
  const bool all_live = qb0 + a.qpb <= a.Tq;
  const int p_first = a.q_pos0 + qb0, p_last = a.q_pos0 + last_q;
  auto interior = [&](int k0) {
    return all_live && k0 + kAttKT - 1 <= p_first && (a.window == 0 || p_last - k0 < a.window);
  };

  const int n_it = (t_end - t_begin + KS - 1) / KS;  // iterations, the same for every group
  if (t_begin + grp < t_end) fetch(t_begin + grp);
  for (int it = 0; it < n_it; ++it) {
    const int tile = t_begin + it * KS + grp;
    const bool has = tile < t_end;  // the group's last iteration may have no tile
    __syncthreads();  // the previous tile's LDS reads are done
    if (has) stage();
    __syncthreads();
    if (tile + KS < t_end) fetch(tile + KS);
    if (!has) continue;
    const int k0 = k_lo + tile * kAttKT;
    // S^T: lane holds keys 16 t + 4 q4 + v of this row, t = 0..3
    v4f st[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      st[t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        st[t] = mfma_bf16(*(const v4i*)(ks + (16 * t + lr) * kKStride + 32 * s + 8 * q4), qr[s], st[t]);
    }
    // a tile inside every row's range (all rows live, every key at or before
    // the block's first position and within the window of its last) needs no mask
    float mx = -INFINITY;
    if (interior(k0)) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          st[t][v] *= a.scale_log2;
          mx = fmaxf(mx, st[t][v]);
        }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int kk = k0 + 16 * t + 4 * q4 + v;
          const bool ok = live && kk <= p && (a.window == 0 || p - kk < a.window);
          st[t][v] = ok ? st[t][v] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, st[t][v]);
        }
    }
    mx = max_xor32(max_xor16(mx));
    const float mnew = fmaxf(mrow, mx);
    const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mrow - mnew);
    const float msub = mnew == -INFINITY ? 0.f : mnew;  // all masked so far: every exp2 is of -inf
    float sum = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        st[t][v] = __builtin_amdgcn_exp2f(st[t][v] - msub);
        sum += st[t][v];
      }
    sum = sum_xor32(sum_xor16(sum));
    lrow = lrow * alpha + sum;
    mrow = mnew;
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] *= alpha;
    // O^T += V^T P^T over two 32-key steps: this lane's slots are keys
    // 32 c + 4 q4 + [0, 4) and 32 c + 16 + 4 q4 + [0, 4).  The probabilities
    // enter as two bf16 parts, p = hi + lo (hi = bf16(p), lo = bf16(p - hi)),
    // so the product with v keeps about 16 bits of each p instead of 8.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      v4i ph, pl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t h, l;
        bf16x2_hi_lo(st[2 * c + e / 2][2 * (e % 2)], st[2 * c + e / 2][2 * (e % 2) + 1], h, l);
        ph[e] = (int)h;
        pl[e] = (int)l;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint16_t* vr = vts + (16 * m + lr) * kVStride + 32 * c + 4 * q4;
        const uint2 lo = *(const uint2*)vr, hi = *(const uint2*)(vr + 16);
        const v4i va = {(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
        acc[m] = mfma_bf16(va, ph, acc[m]);
        acc[m] = mfma_bf16(va, pl, acc[m]);
      }
    }
  }

  if constexpr (KS > 1) {
    // merge: groups 1.. leave their states in LDS (over the tile buffers), group
    // 0 adds them in group order: m = max, each state scaled by 2^(m_g - m)
    static_assert(KS == 2, "one partner group");
    static_assert((size_t)NW * 64 * 34 * 4 <= sizeof(lds), "merge buffer fits the tile buffers");
    const int li = wave * 64 + lane;
    float* mb = (float*)lds + (size_t)li * 32;            // this lane's 32 outputs (16-byte aligned)
    float* ml = (float*)lds + (size_t)NW * 64 * 32 + 2 * li;  // its row's max and sum
    __syncthreads();  // every tile read is done
    if (grp == 1) {
#pragma unroll
      for (int m = 0; m < 8; ++m) *(v4f*)(mb + 4 * m) = acc[m];
      ml[0] = mrow;
      ml[1] = lrow;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = ml[0], l1 = ml[1];
    const float mm = fmaxf(mrow, m1);
    const float a0 = mrow == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrow - mm);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = acc[m] * a0 + *(const v4f*)(mb + 4 * m) * a1;
    lrow = lrow * a0 + l1 * a1;
    mrow = mm;
  }
  // lane holds O^T[d = 16 m + 4 q4 + v][row]; four lanes of a column share the row
  if (!live) return;
  const size_t orow = (size_t)qi * a.Hq + head;
  if (a.n_split == 1) {
    const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      uint2 pk;
      pk.x = bf16x2(acc[m][0] * inv, acc[m][1] * inv);
      pk.y = bf16x2(acc[m][2] * inv, acc[m][3] * inv);
      *(uint2*)(a.o + orow * kAttD + 16 * m + 4 * q4) = pk;
    }
  } else {
    const size_t prow = (size_t)blockIdx.z * a.Tq * a.Hq + orow;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      *(float4*)(a.part_o + prow * kAttD + 16 * m + 4 * q4) = make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
    if (q4 == 0) *(float2*)(a.part_ml + prow * 2) = make_float2(mrow, lrow);
  }
}

// Merge the splits of one (query, head) row: one block per row, one memory
// round trip per phase.  Thread t holds the (max, sum) pairs of splits t and
// t + 256 (fixed-order reductions give the row's maximum M and weighted sum
// L, each split weighted by 2^(m_s - M)); then thread t sums output elements
// 4 (t % 32) .. +3 over the splits s = t / 32 (mod 8), sixteen loads issued
// before the first is used, and the eight partial sums are added in a fixed
// order.
__global__ __launch_bounds__(256) void attention_combine_kernel(AttnArgs a) {
  static_assert(kAttSplitMax <= 512 && kAttD == 128, "two splits per thread, 32 x 4 output elements");
  __shared__ float wsh[kAttSplitMax];
  __shared__ float red[4];
  __shared__ float4 osum[8][32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = a.n_split;
  const int64_t rows = (int64_t)a.Tq * a.Hq;
  const int64_t r = blockIdx.x;
  float2 ml[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sp = tid + 256 * u;
    ml[u] = sp < n ? *(const float2*)(a.part_ml + ((size_t)sp * rows + r) * 2) : make_float2(-INFINITY, 0.f);
  }
  float M = fmaxf(ml[0].x, ml[1].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, kWave));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float L = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int sp = tid + 256 * u;
    const float w = ml[u].x == -INFINITY ? 0.f : exp2f(ml[u].x - M);
    if (sp < n) wsh[sp] = w;
    L += ml[u].y * w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, kWave);
  if (lane == 0) red[wave] = L;
  __syncthreads();
  L = (red[0] + red[1]) + (red[2] + red[3]);
  const int g = tid >> 5, c = tid & 31;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int NB = 16;  // loads in flight per thread: splits g + 8 i, i < NB, per batch
  for (int s0 = g; s0 < n; s0 += 8 * NB) {
    float4 o[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)  // clamped to the last split: unconditional, all issued first
      o[i] = *(const float4*)(a.part_o + ((size_t)min(s0 + 8 * i, n - 1) * rows + r) * kAttD + 4 * c);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float w = s0 + 8 * i < n ? wsh[s0 + 8 * i] : 0.f;
      acc.x += o[i].x * w;
      acc.y += o[i].y * w;
      acc.z += o[i].z * w;
      acc.w += o[i].w * w;
    }
  }
  osum[g][c] = acc;
  __syncthreads();
  if (tid < 32) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      auto e = [&](int gg) { return ((const float*)&osum[gg][c])[i]; };
      v[i] = (((e(0) + e(1)) + (e(2) + e(3))) + ((e(4) + e(5)) + (e(6) + e(7)))) * inv;
    }
    uint2 pk;
    pk.x = bf16x2(v[0], v[1]);
    pk.y = bf16x2(v[2], v[3]);
    *(uint2*)(a.o + r * kAttD + 4 * c) = pk;
  }
}

// Launch plan shared by the workspace query and the launch: query blocks,
// the largest block key range in tiles, and the split of that range.
struct AttnPlan {
  int nw, ks, qpb, q_blocks, max_tiles, n_split, tps;
};

AttnPlan attn_plan(const moe_attn_shape& s, int Tq, int q_pos0) {
  AttnPlan P;
  const int G = s.n_q_heads / s.n_kv_heads;
  P.nw = Tq >= 512 && (2 * kAttRows) % G == 0 ? 8 : 4;  // long query batches: 128-row blocks
  P.qpb = P.nw * 16 / G;
  P.q_blocks = (Tq + P.qpb - 1) / P.qpb;
  // the widest block: a window's block spans window + qpb - 1 keys; the whole
  // context's last block spans every key up to the last query
  const int span = s.window > 0 ? min(s.window + P.qpb - 1, q_pos0 + Tq) : q_pos0 + Tq;
  P.max_tiles = (span + kAttKT - 1) / kAttKT;
  const int base = P.q_blocks * s.n_kv_heads;
  P.n_split = 1;
  if (base < 256) P.n_split = max(1, min(P.max_tiles, (512 + base - 1) / base));  // short batches: ~512 blocks
  P.n_split = min(P.n_split, kAttSplitMax);
  P.tps = (P.max_tiles + P.n_split - 1) / P.n_split;
  P.n_split = (P.max_tiles + P.tps - 1) / P.tps;
  // two key groups per block where a long batch's blocks span many tiles
  // (measured: whole-context prefill chunk of 2048 queries 160 -> 146 us; a
  // 513-key window's ~9 tiles gain nothing and pay the merge)
  P.ks = P.nw == 8 && P.tps >= 16 ? 2 : 1;
  return P;
}

size_t attn_ws_bytes(const moe_attn_shape& s, int Tq, int q_pos0) {
  const AttnPlan P = attn_plan(s, Tq, q_pos0);
  if (P.n_split == 1) return 0;
  const size_t rows = (size_t)Tq * s.n_q_heads;
  return ((size_t)P.n_split * rows * kAttD * 4 + 255) / 256 * 256 + (size_t)P.n_split * rows * 8;
}

hipError_t launch_rope(int T, int H, int D, int pos0, float theta, void* x, hipStream_t st) {
  const double lt = log2((double)theta);
  if ((D / 2) % 4 == 0 && ((uintptr_t)x & 7) == 0) rope_kernel<4><<<(unsigned)T, 256, 0, st>>>((uint16_t*)x, H, D, pos0, lt);
  else rope_kernel<1><<<(unsigned)T, 256, 0, st>>>((uint16_t*)x, H, D, pos0, lt);
  return hipGetLastError();
}

hipError_t launch_attention(const moe_attn_shape& s, int Tq, int Tk, int q_pos0, const void* q, const void* k,
                            const void* v, void* o, void* ws, hipStream_t st) {
  const AttnPlan P = attn_plan(s, Tq, q_pos0);
  AttnArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.Tq = Tq;
  a.Tk = Tk;
  a.Hq = s.n_q_heads;
  a.Hkv = s.n_kv_heads;
  a.G = s.n_q_heads / s.n_kv_heads;
  a.qpb = P.qpb;
  a.q_pos0 = q_pos0;
  a.window = s.window;
  a.n_split = P.n_split;
  a.tps = P.tps;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kAttD));
  const size_t rows = (size_t)Tq * s.n_q_heads;
  a.part_o = P.n_split > 1 ? (float*)ws : nullptr;
  a.part_ml = P.n_split > 1 ? (float*)((char*)ws + ((size_t)P.n_split * rows * kAttD * 4 + 255) / 256 * 256)
                            : nullptr;
  const dim3 grid(P.q_blocks, s.n_kv_heads, P.n_split);
  if (P.nw == 8 && P.ks == 2) attention_kernel<8, 2><<<grid, 1024, 0, st>>>(a);
  else if (P.nw == 8) attention_kernel<8, 1><<<grid, 512, 0, st>>>(a);
  else attention_kernel<4, 1><<<grid, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || P.n_split == 1) return e;
  attention_combine_kernel<<<(unsigned)rows, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe

// ---------------------------------------------------------------------------
// C ABI (include/moe_attn.h)
// ---------------------------------------------------------------------------
extern "C" {

static int attn_status(hipError_t e) { return e == hipSuccess ? MOE_ATTN_OK : MOE_ATTN_ERR_HIP; }

static int attn_validate(const moe_attn_shape* s, int32_t Tq, int32_t Tk, int32_t q_pos0) {
  if (!s || Tq < 0 || Tk < 0 || q_pos0 < 0 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->window < 0)
    return MOE_ATTN_ERR_INVALID_ARG;
  if (s->n_q_heads % s->n_kv_heads || (int64_t)q_pos0 + Tq > Tk) return MOE_ATTN_ERR_INVALID_ARG;
  const int G = s->n_q_heads / s->n_kv_heads;
  if (s->head_dim != moe::kAttD || moe::kAttRows % G || s->n_kv_heads > 65535) return MOE_ATTN_ERR_UNSUPPORTED;
  if ((int64_t)Tk * s->n_kv_heads * moe::kAttD >= (int64_t)1 << 40) return MOE_ATTN_ERR_UNSUPPORTED;
  return MOE_ATTN_OK;
}

int moe_rope(int32_t T, int32_t n_heads, int32_t head_dim, int32_t pos0, float theta, void* x, void* stream) {
  if (T < 0 || n_heads < 1 || head_dim < 2 || head_dim % 2 || head_dim > 1024 || pos0 < 0 || !(theta > 1.0f))
    return MOE_ATTN_ERR_INVALID_ARG;
  if (T == 0) return MOE_ATTN_OK;
  if (!x) return MOE_ATTN_ERR_INVALID_ARG;
  if ((int64_t)n_heads * (head_dim / 2) >= INT32_MAX) return MOE_ATTN_ERR_UNSUPPORTED;
  return attn_status(moe::launch_rope(T, n_heads, head_dim, pos0, theta, x, (hipStream_t)stream));
}

size_t moe_attn_workspace_bytes(const moe_attn_shape* s, int32_t Tq, int32_t Tk, int32_t q_pos0) {
  if (attn_validate(s, Tq, Tk, q_pos0) != MOE_ATTN_OK) return 0;
  return moe::attn_ws_bytes(*s, Tq, q_pos0);
}

int moe_attention(const moe_attn_shape* s, int32_t Tq, int32_t Tk, int32_t q_pos0, const void* q, const void* k,
                  const void* v, void* o, void* ws, size_t ws_bytes, void* stream) {
  const int rc = attn_validate(s, Tq, Tk, q_pos0);
  if (rc != MOE_ATTN_OK) return rc;
  if (Tq == 0) return MOE_ATTN_OK;
  if (!q || !k || !v || !o) return MOE_ATTN_ERR_INVALID_ARG;
  const size_t need = moe::attn_ws_bytes(*s, Tq, q_pos0);
  if (need > 0 && !ws) return MOE_ATTN_ERR_INVALID_ARG;
  if (ws_bytes < need) return MOE_ATTN_ERR_WORKSPACE;
  return attn_status(moe::launch_attention(*s, Tq, Tk, q_pos0, q, k, v, o, ws, (hipStream_t)stream));
}

}  // extern "C"
