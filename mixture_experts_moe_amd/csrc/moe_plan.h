// The dispatch plan: everything the expert kernels need to find their work,
// built by the routing call's last launch.
//  * Block schedules of the two expert kernels.  Tiles: per group (routed
//    experts 0..E-1, then the shared expert with all T rows) ceil(rows / BM)
//    tiles of BM rows, in group order; work item i = tile * n_slices + slice.
//    Block b of a kernel gets item i = b (identity), or, in XCD mode, item
//    (b % 8) * L + b / 8 with L = ceil(items / 8): the chip's eight XCDs (block
//    b runs on XCD b % 8, each with its own L2) then each take one contiguous
//    run of items, so the tiles of one expert run on one XCD close together in
//    time and share its weight stream through that L2.  A record is (group,
//    first row, first h row, rows | slice << 16), or group -1 for a block
//    without work.
//  * Per h row q (sorted pairs, then P + t for the shared expert): token,
//    partial-output row and routing weight.
//  * With FP8 weights, the activations as E4M3 codes with per-(token, 128)
//    scales.
//  * For tile-list plans, two counters per tile that the fused expert launch
//    synchronises on (zeroed here; the launch leaves them zero).
#pragma once

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// Activation quantisation of 128-element groups by one wave: per group
// s = amax/448 (1 for an all-zero group), code = E4M3(v/s), round to nearest
// even, saturating.  The wave takes four groups at a time, one per 16 lanes,
// eight elements per lane (one 16-byte load, one 8-byte store): groups
// g0 .. g0+3 of row `row` (those below gpr, the groups per row).
template <bool BF16IN>
__device__ __forceinline__ void quantize_groups4(const void* __restrict__ in, int64_t row, int g0, int gpr,
                                                 uint8_t* __restrict__ codes, float* __restrict__ scales, int lane) {
  const int g = g0 + (lane >> 4), l16 = lane & 15;
  if (g < gpr) {  // whole 16-lane groups drop out together
    const int64_t o = (row * gpr + g) * 128 + 8 * l16;
    float v[8];
    if (BF16IN) {
      const v4i pr = *(const v4i*)((const uint16_t*)in + o);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float((uint32_t)pr[i] << 16);
        v[2 * i + 1] = __uint_as_float((uint32_t)pr[i] & 0xffff0000u);
      }
    } else {
      const float4 a = *(const float4*)((const float*)in + o), b = *(const float4*)((const float*)in + o + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) m = fmaxf(m, __shfl_xor(m, x, kWave));
    const float s = m > 0.f ? m / 448.0f : 1.0f;
    uint2 c;
    c.x = pack4_e4m3(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
    c.y = pack4_e4m3(v[4] / s, v[5] / s, v[6] / s, v[7] / s);
    *(uint2*)(codes + o) = c;
    if (l16 == 0) scales[row * gpr + g] = s;
  }
}

// A whole row by one wave.
template <bool BF16IN>
__device__ __forceinline__ void quantize_row(const void* __restrict__ in, int64_t row, int gpr,
                                             uint8_t* __restrict__ codes, float* __restrict__ scales, int lane) {
  for (int g0 = 0; g0 < gpr; g0 += 4) quantize_groups4<BF16IN>(in, row, g0, gpr, codes, scales, lane);
}

// Group tables of one plan block: tile prefix, rows and first h row per group.
struct PlanLds {
  int32_t tstart[kMaxExperts + 2], grow[kMaxExperts + 1], gh0[kMaxExperts + 1], tmp[17];
};

// Fills the tables (every thread of an NT-thread block takes part); returns the
// number of tiles.  Ends with a barrier.
template <int NT>
__device__ int plan_tables(const PlanArgs& pa, PlanLds& L) {
  constexpr int PER = (kMaxExperts + 1 + NT - 1) / NT;  // groups per thread
  const int E = pa.E, G = E + (pa.has_shared ? 1 : 0), BM = pa.BM;
  int nt[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = PER * threadIdx.x + i;
    const int rows = g < E ? pa.counts[g] : (g < G ? pa.T : 0);
    if (g < G) {
      L.grow[g] = rows;
      L.gh0[g] = g < E ? pa.offsets[g] : pa.P;
    }
    nt[i] = (rows + BM - 1) / BM;
    sum += nt[i];
  }
  int total;
  int st = block_excl_scan<NT>(sum, L.tmp, &total);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int g = PER * threadIdx.x + i;
    if (g < G) L.tstart[g] = st;
    st += nt[i];
  }
  if (threadIdx.x == 0) L.tstart[G] = total;
  __syncthreads();
  return total;
}

// Tile-list entry t (identity schedules) of a plan with `total` tiles.
__device__ __forceinline__ void plan_tile_entry(const PlanArgs& pa, const PlanLds& L, int total, int t) {
  if (t >= pa.max_tiles) return;
  if (pa.sync) pa.sync[t] = pa.sync[pa.max_tiles + t] = 0;
  int4 rec = make_int4(-1, 0, 0, 0);
  if (t < total) {
    const int G = pa.E + (pa.has_shared ? 1 : 0);
    int lo = 0, hi = G - 1;  // the last group whose first tile is <= t (it has tiles)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (L.tstart[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int m0 = (t - L.tstart[lo]) * pa.BM;
    rec = make_int4(lo, m0, L.gh0[lo] + m0, min(pa.BM, L.grow[lo] - m0));
  }
  pa.sched[0][t] = rec;
}

// Number of plan entries a plan writes: the tile list, or one record per block
// of each kernel (XCD schedules).
__device__ __host__ inline int plan_n_entries(const PlanArgs& pa) {
  return pa.xcd ? pa.n_sched[0] + pa.n_sched[1] : pa.max_tiles;
}

// Plan entry e: a tile-list entry, or (XCD) a block record.
__device__ __forceinline__ void plan_any_entry(const PlanArgs& pa, const PlanLds& L, int total, int e);

// Schedule entry e (gate/up entries first, then down) of a plan with `total` tiles.
__device__ __forceinline__ void plan_entry(const PlanArgs& pa, const PlanLds& L, int total, int e) {
  const int which = e < pa.n_sched[0] ? 0 : 1;
  const int b = which ? e - pa.n_sched[0] : e;
  if (b >= pa.n_sched[which]) return;
  const int nsl = pa.n_slices[which];
  const int n_items = total * nsl;
  int item = b;
  if (pa.xcd) {
    const int Lr = (n_items + 7) / 8, j = b / 8;
    item = j < Lr ? (b % 8) * Lr + j : n_items;
  }
  int4 rec = make_int4(-1, 0, 0, 0);
  if (item < n_items) {
    const int t = item / nsl, sl = item - t * nsl;
    const int G = pa.E + (pa.has_shared ? 1 : 0);
    int lo = 0, hi = G - 1;  // the last group whose first tile is <= t (it has tiles)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (L.tstart[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int m0 = (t - L.tstart[lo]) * pa.BM;
    rec = make_int4(lo, m0, L.gh0[lo] + m0, min(pa.BM, L.grow[lo] - m0) | (sl << 16));
  }
  pa.sched[which][b] = rec;
}

__device__ __forceinline__ void plan_any_entry(const PlanArgs& pa, const PlanLds& L, int total, int e) {
  if (pa.xcd) plan_entry(pa, L, total, e);
  else plan_tile_entry(pa, L, total, e);
}

// Schedule build by groups, for one block (short inputs): thread tid owns
// groups PER*tid .. PER*tid + PER-1 (as in plan_tables) and writes every record
// of their tiles at its block position -- identity, or in XCD mode the inverse
// of item = (b % 8) * L + b / 8, b = (item % L) * 8 + item / L -- then the
// positions no item maps to get group -1.  No search per record.
template <int NT>
__device__ void plan_scatter(const PlanArgs& pa, const PlanLds& L, int total) {
  constexpr int PER = (kMaxExperts + 1 + NT - 1) / NT;
  const int G = pa.E + (pa.has_shared ? 1 : 0), BM = pa.BM;
  if (!pa.xcd) {  // the tile list only
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = PER * threadIdx.x + i;
      if (g >= G) break;
      const int t0 = L.tstart[g], nt = L.tstart[g + 1] - t0;
      for (int j = 0; j < nt; ++j)
        pa.sched[0][t0 + j] = make_int4(g, j * BM, L.gh0[g] + j * BM, min(BM, L.grow[g] - j * BM));
    }
    for (int t = total + threadIdx.x; t < pa.max_tiles; t += NT) pa.sched[0][t] = make_int4(-1, 0, 0, 0);
    if (pa.sync)
      for (int t = threadIdx.x; t < 2 * pa.max_tiles; t += NT) pa.sync[t] = 0;
    return;
  }
  for (int which = 0; which < 2; ++which) {
    const int nsl = pa.n_slices[which], n_items = total * nsl, Lr = (n_items + 7) / 8;
    int4* sched = pa.sched[which];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int g = PER * threadIdx.x + i;
      if (g >= G) break;
      const int t0 = L.tstart[g], nt = L.tstart[g + 1] - t0;
      for (int j = 0; j < nt; ++j) {
        const int m0 = j * BM, rows = min(BM, L.grow[g] - m0);
        for (int sl = 0; sl < nsl; ++sl) {
          const int item = (t0 + j) * nsl + sl;
          const int b = pa.xcd ? (item % Lr) * 8 + item / Lr : item;
          sched[b] = make_int4(g, m0, L.gh0[g] + m0, rows | (sl << 16));
        }
      }
    }
    for (int b = threadIdx.x; b < pa.n_sched[which]; b += NT) {
      const int item = pa.xcd ? ((b / 8) < Lr ? (b % 8) * Lr + b / 8 : n_items) : b;
      if (item >= n_items) sched[b] = make_int4(-1, 0, 0, 0);
    }
  }
}

}  // namespace moe
