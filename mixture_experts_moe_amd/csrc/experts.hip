// Expert kernels: activation quantisation, tile planning, grouped gate/up and
// down projections (FP8 E4M3 and bf16 on the gfx950 matrix cores, fp32 plain),
// and the fixed-order weighted combine.
//
// Pages cited by title and section:
//   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
//   [cache] "Kolibri-1 CPU dequant cache" (vllm.cpp pull request 3488)
//
// The layer ([port] "The gate"): each token runs through its k routed experts
// and one shared expert; the expert layer is a gated linear unit ([port] part
// 3), here SwiGLU: h = silu(W_gate x) * (W_up x), y = W_down h.  The expert
// weights are FP8 codes decoded for compute ([cache], first paragraph): here the
// matrix cores consume the codes directly and the fp32 block scales are applied
// to each 128-deep partial product in registers, so no decoded copy of a weight
// ever exists.
//
// Grouped GEMM layout.  Group g < E is routed expert g, whose rows are the pairs
// q in [offsets[g], offsets[g+1]) in sorted order; group E is the shared expert,
// whose rows are the tokens 0..T-1.  A tile is (group, first row m0) covering up
// to BM rows; a block computes one tile against one slice of output features:
// weights stream from HBM straight into matrix-core operand registers (each
// weight byte is read once per tile), while the tile's activation rows sit in
// LDS for the whole K loop.
#include <limits.h>

#include "moe.h"
#include "moe_device.h"
#include "moe_kernels.h"
#include "moe_plan.h"

namespace moe {

#ifndef MOE_GU_KG
#define MOE_GU_KG 4  // K blocks per weight stage in the gate/up stream (16-row tiles)
#endif
#ifndef MOE_GU_KG_TALL
#define MOE_GU_KG_TALL 2  // the same for taller tiles, split between gate and up (4 spills past
                          // 128 registers: one block per CU instead of two, measured slower)
#endif

// Load of 16 weight bytes.  NT: non-temporal, for launches that read each
// expert's weights once (FP8 weights in 16-row tiles: identity block schedule,
// chosen when experts average at most 12 rows, so one tile per expert in the
// usual case).  Measured on MI355X at decode, the streaming hint
// keeps the weight stream from evicting the small outputs the kernels write
// (h codes, fp32 partials) and the activations they re-read, whose dirty lines
// otherwise go back to HBM in the middle of the stream: gate/up -3 us, down
// -4.5 us per launch.  Taller tiles (XCD schedules) read an expert's weights
// once per row tile and rely on L2 keeping them between the tiles, so they use
// ordinary loads.
template <bool NT>
__device__ __forceinline__ v4i stream_load(const uint8_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load((const v4i*)p);
  else return *(const v4i*)p;
}

// ---------------------------------------------------------------------------
// Activation quantisation on its own (moe_quantize_rows): one wave per row, as
// in the routing call's plan step.
// ---------------------------------------------------------------------------
template <bool BF16IN>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* __restrict__ in, int64_t n_rows, int gpr,
                                                             uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  quantize_row<BF16IN>(in, row, gpr, codes, scales, threadIdx.x & 63);
}

// Address of the weight bytes a lane streams for one 16-row tile: in the
// row-major layout lane l reads row (16*rt + l%16) at byte 16*(l/16) of each
// 128-byte K block (and 64 further for the upper half); in the tiled layout the
// same bytes sit at 16*l of the tile's 2 KB (upper half: +1024).
// The stream goes through a buffer resource over the wave's n16 tiles of 16
// rows (base and size wave-uniform): the lane's byte offset is fixed and the K
// block's offset is a scalar, so a load costs no vector address arithmetic.
// Offsets past the resource's size would read zeros, never another buffer.
struct WeightStream {
  __amdgpu_buffer_rsrc_t r;  // the wave's rows
  int voff;                  // this lane's first byte in K block 0 of its first tile
  int kb_stride;             // bytes from one K block to the next
  int hi_off;                // bytes from the lower to the upper 64-byte half
  int tile_step;             // bytes from one 16-row tile to the next
};
__device__ __forceinline__ WeightStream weight_stream(const uint8_t* mat, int row_bytes, int row0, bool tiled,
                                                      int lane, int n16 = 1) {
  WeightStream w;
  const uint8_t* base = mat + (size_t)row0 * row_bytes;  // the tiled layout keeps a 16-row tile's bytes together
  w.r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, n16 * 16 * row_bytes, 0x00020000);
  if (tiled) {
    w.voff = lane * 16;
    w.kb_stride = 2048;
    w.hi_off = 1024;
    w.tile_step = (row_bytes / 128) * 2048;
  } else {
    w.voff = (lane & 15) * row_bytes + (lane >> 4) * 16;
    w.kb_stride = 128;
    w.hi_off = 64;
    w.tile_step = 16 * row_bytes;
  }
  return w;
}
// 16 bytes of the stream at scalar offset soff; NT: non-temporal.
template <bool NT>
__device__ __forceinline__ v4i stream_load(const WeightStream& w, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(w.r, w.voff, soff, NT ? 2 : 0));
}
// A buffer resource over `bytes` bytes from a wave-uniform base, and 16- and
// 8-byte loads at a lane offset plus a scalar offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}
template <bool NT>
__device__ __forceinline__ v4i buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0));
}
__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// Rows of one tile: for each of its BM rows, the activation (token) row, the
// output row of h (sorted pair index, or P + t for the shared expert), the
// partial-output row (pair index p, or P + t) and the routing weight.
struct TileRows {
  int g, m0, hrow0, rows;  // g < 0: no tile
  bool shared;
};

// The block's schedule record (written by the plan step): its tile's rows and
// its feature slice.
__device__ __forceinline__ TileRows block_rows(const ExpertArgs& a, int b, int& slice) {
  int4 rec;
  if (a.per_tile) {
    rec = a.sched[b / a.nsl];
    slice = b % a.nsl;
  } else {
    rec = a.sched[b];
    slice = rec.w >> 16;
  }
  TileRows r;
  r.g = rec.x;
  r.m0 = rec.y;
  r.hrow0 = rec.z;
  r.rows = rec.w & 0xffff;
  r.shared = rec.x == a.E;
  return r;
}

// ---------------------------------------------------------------------------
// Gate/up projection + SwiGLU epilogue on the matrix cores.
//   WT = 2: FP8 E4M3 weights and activation codes streamed as bytes; each
//           128-deep K block is one exactly-accumulated product of the codes
//           (kblock_e4m3_exact), then partial * (s_x[row][kb] * s_w[block][kb])
//           is added in fp32; h quantised per (row, 128-feature group) in the
//           epilogue.
//   WT = 1: bf16 weights and activations, 16x16x32 MFMA accumulating in fp32;
//           h stored as bf16.
// Block = 8 waves covering one 128-feature group nb of h for one tile (see
// block_rows).  Wave w owns h features nb*128 + w*16 + [0, 16): one 16-row
// tile of W_gate and the same rows of W_up, so g and u of a feature meet in one
// lane.  32 weight rows per wave keeps many short streams in flight, which the
// HBM prefers to a few long ones.
// ---------------------------------------------------------------------------
constexpr int kGateUpWaves = 8;

// Taller FP8 tiles stage their activations in LDS as bf16, one part of K at a
// time (K blocks [0, n), then [n, d/128)), so the bf16 row is no wider than
// the row of E4M3 codes it replaces and each activation element is decoded
// once per block rather than once per wave.  n is even: the product loop takes
// its single-block stages in pairs, and the switch falls between two pairs.
__host__ __device__ constexpr int gateup_x_part_blocks(int nkb) { return nkb < 4 ? nkb : (nkb + 3) / 4 * 2; }

// Device-coherent 32-bit store and load (agent-scope relaxed atomics: written
// through to, and read from, the point where all XCDs see the same data), for
// results one block hands to blocks on other XCDs within one launch.
__device__ __forceinline__ void store_coherent(void* p, uint32_t v) {
  __hip_atomic_store((uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_coherent(const void* p) {
  return __hip_atomic_load((const uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The work of gate/up block b (smem: the block's dynamic LDS).  Returns false
// for a block without work.  COH: h codes and scales are stored coherently
// (the fused expert launch).  A16 (with WT = 2): W8A16 -- the activation rows
// are bf16 (not quantised, unit scales) and h is stored as bf16.
// LDS rows of bf16 activations (or h) in the FP8 weight codes' K order,
// arranged so that the four 16-byte fragments a lane reads per 128-element K
// block sit at 16 * (lane / 16) + 64 * i: the 16-element unit u of a row (K
// elements 16u .. 16u + 15) keeps its first 8 elements at xunit_pos(u) and
// the other 8 at xunit_pos(u) + 64.  Each fragment read is then 16 rows x 4
// lanes at 16-byte steps, which with row strides of 32 bytes past a multiple
// of 64 (rows of 2 * 64n + 32 bytes) touches every LDS bank once per group of
// lanes the hardware serves together (measured: 32-byte steps conflict at any
// 16-byte-aligned row stride).
__device__ __forceinline__ int xunit_pos(int u) { return (u >> 3) * 256 + ((u >> 2) & 1) * 128 + (u & 3) * 16; }
constexpr int kLdsRowPad = 32;  // bytes past a row's data: a row stride of 32 modulo 64 bytes

template <int BM, int WT, bool XB, bool COH = false, bool A16 = false>
__device__ __forceinline__ bool gateup_block(const ExpertArgs& a, int b, uint8_t* smem) {
  static_assert(!A16 || (WT == 2 && XB), "W8A16 stages bf16 activations for FP8 weights");
  constexpr bool XQ = WT == 2 && !A16;  // activations as E4M3 codes with scales, h quantised
  constexpr int NC = BM / 16;
  constexpr int EB = WT == 2 ? 1 : 2;   // bytes per weight element
  constexpr int EX = XQ ? 1 : 2;        // bytes per activation element in HBM
  constexpr int NT = kGateUpWaves * 64;
  constexpr bool XBF = WT == 1 || XB;  // whole activation rows in LDS as bf16 (else XH, or E4M3 codes)
  constexpr bool XH = BM > 16 && XQ && !XB;  // bf16 activations in LDS by parts of K (gateup_x_part_blocks)
  int nb;
  const TileRows tr = block_rows(a, b, nb);
  if (tr.g < 0) return false;
  const int Fg = tr.shared ? a.Fs : a.F;
  if (nb * 128 >= Fg) return false;

  const int RB = a.d * EB;        // bytes per weight row in HBM
  const int RX = a.d * EX;        // bytes per activation row in HBM
  const int nbb = RB / 128;       // 128-byte K blocks of a weight row
  const int nkh = XH ? gateup_x_part_blocks(a.d / 128) : a.d / 128;  // K blocks of the first part
  const int xstride = (XH ? nkh * 256 : XBF ? a.d * 2 : a.d) + kLdsRowPad;  // padded LDS row of activations
  uint8_t* xs = smem;
  // [2][d/128][BM] (FP8 only): per matrix (gate, up), K block and row, the
  // activation scale times the weight block scale; one K block's rows adjacent
  float* csc = (float*)(smem + (BM + 1) * xstride);
  float* red = csc + (WT == 2 ? 2 * BM * (a.d / 128) : 0);  // [waves][BM]

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lk = (lane >> 4) * 16;
  const size_t wsz = (size_t)a.F * RB;  // bytes of one routed expert matrix
  const uint8_t* wg = tr.shared ? (const uint8_t*)a.shg : (const uint8_t*)a.wg + (size_t)tr.g * wsz;
  const uint8_t* wu = tr.shared ? (const uint8_t*)a.shu : (const uint8_t*)a.wu + (size_t)tr.g * wsz;
  const int f0 = nb * 128 + wave * 16;
  const WeightStream ws[2] = {weight_stream(wg, RB, f0, a.w_tiled, lane), weight_stream(wu, RB, f0, a.w_tiled, lane)};
  const float* sgp = nullptr;
  const float* sup = nullptr;
  if (WT == 2) {
    const int nkb = a.d / 128;
    const size_t ssz = (size_t)(a.F / 128) * nkb;
    sgp = (tr.shared ? a.ssg : a.sg + (size_t)tr.g * ssz) + (size_t)nb * nkb;
    sup = (tr.shared ? a.ssu : a.su + (size_t)tr.g * ssz) + (size_t)nb * nkb;
  }

  v4f acc[2][NC];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};

  // Weight stream.  Stage = KG consecutive K blocks of one 16-row tile (gate
  // or up); two register slots, two stages in flight.
  //  * 16-row tiles (SEQ): the wave reads its gate tile over all of K, then its
  //    up tile -- one long run after the other streams faster than the two
  //    interleaved (measured).  Stage st < nq is gate group st, otherwise up
  //    group st - nq; the slots take alternate stages.
  //  * Taller tiles: stage st = group st of KG/2 K blocks of both tiles (gate
  //    blocks in register entries [0, KG/2), up blocks in [KG/2, KG)), so that
  //    each activation chunk, decoded from its E4M3 codes, serves both
  //    products; the sequential order spills there.
  // The loop bodies issue their loads unconditionally (a short last group
  // re-reads the final K block, in bounds and in cache) and the last pair of
  // stages is peeled, so the memory-counter waits stay exact and nothing is
  // fetched twice in the steady state.  Slots and tiles are template constants
  // (Ic), so the register arrays are never indexed at run time.
  constexpr bool SEQ = BM == 16;
  constexpr int KG = SEQ ? MOE_GU_KG : MOE_GU_KG_TALL;
  constexpr int KGP = KG / 2;  // blocks per tile in a taller-tile stage
  static_assert(SEQ || (KG % 2 == 0 && WT == 2 && !XB), "taller tiles: FP8 weights, a stage split between the tiles");
  const int nq = SEQ ? (nbb + KG - 1) / KG : (nbb + KGP - 1) / KGP;
  const int ns = SEQ ? 2 * nq : nq;
  v4i wlo[2][KG], whi[2][KG];
  auto load = [&](auto S, int st) {
    constexpr int sl = decltype(S)::value;
    if constexpr (SEQ) {
      const bool up = st >= nq;
      const int q = up ? st - nq : st;
      const WeightStream& w = ws[up ? 1 : 0];
#pragma unroll
      for (int j = 0; j < KG; ++j) {
        const int so = min(q * KG + j, nbb - 1) * ws[0].kb_stride;
        wlo[sl][j] = stream_load<WT == 2>(w, so);
        whi[sl][j] = stream_load<WT == 2>(w, so + ws[0].hi_off);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < KGP; ++j) {
          const int so = min(st * KGP + j, nbb - 1) * ws[0].kb_stride;
          wlo[sl][m * KGP + j] = stream_load<false>(ws[m], so);
          whi[sl][m * KGP + j] = stream_load<false>(ws[m], so + ws[0].hi_off);
        }
    }
  };
  // Staging.  Loads complete in issue order as far as the wait counter goes,
  // so the order is pinned: the token of each row this thread stages (perm),
  // the activation and weight block scales, then the weight stream, then the
  // activation rows (which need the tokens).  The scale products go to LDS, so
  // the product loop reads no global memory besides the weight stream.
  // All loads are unconditional (clamped addresses) and the chunks past the
  // tile land in a spare LDS row, so the code is straight-line and every wait
  // is exact.  The first batch of SB chunks per thread covers a
  // 16-row tile at d = 2048, and one part of a 32-row tile (XH).
  // XH: part 0 of the rows is staged here, part 1 between two barriers when
  // the products reach it (next_part).
  constexpr int SB = 4;
  const int cpr = RX / 16, nkb = a.d / 128;
  const int cps0 = XH ? nkh * 8 : cpr, cps1 = XH ? max(cpr - cps0, 1) : 1;  // chunks per row of part 0, 1
  const uint8_t* xa = (const uint8_t*)a.xa;
  const int rlast = tr.rows - 1;
  auto row_token = [&](int r) { return a.ri.tok[tr.hrow0 + min(r, rlast)]; };  // token of tile row r (clamped)
  // Chunk i of a part (cps chunks per row) is chunk i % cps of row i / cps.  A
  // thread's batch is chunks i0 + u*NT, whose row and chunk advance by NT / cps
  // and NT % cps: one division per batch rather than two per chunk.
  struct Batch {
    int r[SB], c[SB];
  };
  auto chunk_walk = [&](int i0, int part) {
    const int cps = part ? cps1 : cps0;
    const int dr = NT / cps, dc = NT - dr * cps;
    int r = i0 / cps, c = i0 - r * cps;
    Batch bt;
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      bt.r[u] = r;
      bt.c[u] = c;
      r += dr;
      c += dc;
      const bool wrap = c >= cps;
      r += wrap ? 1 : 0;
      c -= wrap ? cps : 0;
    }
    return bt;
  };
  auto chunk_tokens = [&](const Batch& bt, int (&tk)[SB]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) tk[u] = row_token(bt.r[u]);
  };
  auto chunk_load = [&](const Batch& bt, int part, const int (&tk)[SB], v4i (&v)[SB]) {
    const int c0 = part ? cps0 : 0;
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int c = min(c0 + bt.c[u], cpr - 1);  // clamped: in bounds
      v[u] = *(const v4i*)(xa + (size_t)tk[u] * RX + c * 16);
    }
  };
  // Rows past the tile (r > rlast) hold copies of the last row (row_token
  // clamps): their products are never stored, and no output row reads another
  // row's activations.  Chunks past the part's last row (r >= BM) go to the
  // spare row.
  auto chunk_store = [&](const Batch& bt, const v4i (&v)[SB]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int r = bt.r[u];
      const bool in = r < BM;
      const v4i x = v[u];
      uint8_t* dst = xs + (in ? r : BM) * xstride;
      const int c = in ? bt.c[u] : 0;
      if constexpr (XQ && (XB || XH)) {  // E4M3 codes -> bf16 once per block (exact)
        v4i lo, hi;
        e4m3x16_to_bf16(x, lo, hi);
        *(v4i*)(dst + xunit_pos(c)) = lo;
        *(v4i*)(dst + xunit_pos(c) + 64) = hi;
      } else if constexpr (WT == 2 && XBF) {  // bf16 activations (W8A16): 8 elements of a unit
        *(v4i*)(dst + xunit_pos(c >> 1) + 64 * (c & 1)) = x;
      } else {
        *(v4i*)(dst + c * 16) = x;
      }
    }
  };
  {
    int tk[SB];
    const Batch bt = chunk_walk(tid, 0);
    chunk_tokens(bt, tk);
    float sv = 0.f, gv = 0.f, uv = 0.f;
    if (WT == 2) {  // row tid % BM, K block tid / BM (clamped: in bounds)
      const int kb = min(tid / BM, nkb - 1);
      sv = XQ ? a.sxa[(size_t)row_token(tid % BM) * nkb + kb] : 1.0f;
      gv = sgp[kb];  // the slice's weight block scales
      uv = sup[kb];
    }
    __builtin_amdgcn_sched_barrier(0);
    load(Ic<0>{}, 0);
    load(Ic<1>{}, 1);
    __builtin_amdgcn_sched_barrier(0);
    v4i v[SB];
    chunk_load(bt, 0, tk, v);
    chunk_store(bt, v);
    if (WT == 2 && tid < BM * nkb) {
      const float sx = tid % BM <= rlast ? sv : 0.f;
      csc[tid] = sx * gv;
      csc[BM * nkb + tid] = sx * uv;
    }
  }
  for (int i0 = tid + NT * SB; i0 < BM * cps0; i0 += NT * SB) {  // tall tiles or wide rows only
    int tk[SB];
    v4i v[SB];
    const Batch bt = chunk_walk(i0, 0);
    chunk_tokens(bt, tk);
    chunk_load(bt, 0, tk, v);
    chunk_store(bt, v);
  }
  if (WT == 2) {
    for (int i = tid + NT; i < BM * nkb; i += NT) {  // tall tiles or wide rows only
      const float sx = i % BM <= rlast ? (XQ ? a.sxa[(size_t)row_token(i % BM) * nkb + i / BM] : 1.0f) : 0.f;
      csc[i] = sx * sgp[i / BM];
      csc[BM * nkb + i] = sx * sup[i / BM];
    }
  }
  __syncthreads();
  // XH: every wave is past part 0's products; part 1 replaces it in LDS
  auto next_part = [&]() {
    __syncthreads();
    for (int i0 = tid; i0 < BM * cps1; i0 += NT * SB) {
      int tk[SB];
      v4i v[SB];
      const Batch bt = chunk_walk(i0, 1);
      chunk_tokens(bt, tk);
      chunk_load(bt, 1, tk, v);
      chunk_store(bt, v);
    }
    __syncthreads();
  };

  auto compute_run = [&](auto R, auto S, int q) {
    constexpr int r = decltype(R)::value, sl = decltype(S)::value;
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const int bb = q * KG + j;
      if (bb >= nbb) break;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (WT == 2) {
          v4i b[4];
          if constexpr (XB) {
            // bf16 activations of K block bb in the weight codes' K order: codes
            // 16*(lane/16) + [0,16) of each 64-element half (xunit_pos layout)
            const uint8_t* bp = xs + (c * 16 + lr) * xstride + bb * 256 + lk;
            b[0] = *(const v4i*)bp;
            b[1] = *(const v4i*)(bp + 64);
            b[2] = *(const v4i*)(bp + 128);
            b[3] = *(const v4i*)(bp + 192);
          } else {  // codes, decoded here
            const uint8_t* bp = xs + (c * 16 + lr) * xstride + bb * 128 + lk;
            e4m3x16_to_bf16(*(const v4i*)bp, b[0], b[1]);
            e4m3x16_to_bf16(*(const v4i*)(bp + 64), b[2], b[3]);
          }
          acc[r][c] += kblock_e4m3_exact(wlo[sl][j], whi[sl][j], b) * csc[(r * nbb + bb) * BM + c * 16 + lr];
        } else {
          const uint8_t* bp = xs + (c * 16 + lr) * xstride + bb * 128 + lk;
          const v4i blo = *(const v4i*)bp;
          const v4i bhi = *(const v4i*)(bp + 64);
          acc[r][c] = mfma_bf16(wlo[sl][j], blo, acc[r][c]);
          acc[r][c] = mfma_bf16(whi[sl][j], bhi, acc[r][c]);
        }
      }
    }
  };
  // taller tiles: both tiles' blocks of group q; each activation chunk and each
  // weight block decoded from its E4M3 codes once (XH: the activations were
  // decoded when staged)
  auto compute_pair = [&](auto S, int q) {
    constexpr int sl = decltype(S)::value;
#pragma unroll
    for (int j = 0; j < KGP; ++j) {
      const int bb = q * KGP + j;
      if (bb >= nbb) break;
      v4i b[NC][4];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (XH) {  // bf16, in the weight codes' K order (as for XB)
          const int bl = bb < nkh ? bb : bb - nkh;  // K block within the staged part
          const uint8_t* bp = xs + (c * 16 + lr) * xstride + bl * 256 + lk;
          b[c][0] = *(const v4i*)bp;
          b[c][1] = *(const v4i*)(bp + 64);
          b[c][2] = *(const v4i*)(bp + 128);
          b[c][3] = *(const v4i*)(bp + 192);
        } else {
          const uint8_t* bp = xs + (c * 16 + lr) * xstride + bb * 128 + lk;
          e4m3x16_to_bf16(*(const v4i*)bp, b[c][0], b[c][1]);
          e4m3x16_to_bf16(*(const v4i*)(bp + 64), b[c][2], b[c][3]);
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        v4i w[4];
        kblock_decode(wlo[sl][m * KGP + j], whi[sl][m * KGP + j], w);
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[m][c] += kblock_bf16(w, b[c]) * csc[(m * nbb + bb) * BM + c * 16 + lr];
      }
    }
  };
  auto compute = [&](auto S, int st) {
    if constexpr (!SEQ) {
      if constexpr (WT == 2 && !XB) compute_pair(S, st);
    } else if (st < nq) {
      compute_run(Ic<0>{}, S, st);
    } else {
      compute_run(Ic<1>{}, S, st - nq);
    }
  };
  static_assert(!XH || KGP == 1, "the part switch falls on a stage boundary");
  const int st_part = XH && nkh < nkb ? nkh : -1;  // first stage of part 1 (even)
  int st = 0;
  for (; st + 2 < ns; st += 2) {  // both loads of the body are in range
    if (st == st_part) next_part();
    compute(Ic<0>{}, st);
    load(Ic<0>{}, st + 2);
    compute(Ic<1>{}, st + 1);
    load(Ic<1>{}, st + 3);
  }
  if (st == st_part) next_part();
  compute(Ic<0>{}, st);
  if (st + 1 < ns) compute(Ic<1>{}, st + 1);  // taller tiles: the number of groups may be odd

  // Epilogue: h = silu(g) * u for features f0 + 4*(lane/16) + i, row c*16 + lane%16.
  float h[NC][4];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gv = acc[0][c][i], uv = acc[1][c][i];
      h[c][i] = silu_f32(gv) * uv;
    }
  const int hrow0 = tr.hrow0;
  const int fcol = f0 + 4 * (lane >> 4);
  if constexpr (XQ) {  // h quantised per (row, 128 features); else stored as bf16
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(h[c][i]));
      m = max_xor32(max_xor16(m));
      if (lane < 16) red[wave * BM + c * 16 + lane] = m;
    }
    __syncthreads();
    uint8_t* hq = (uint8_t*)a.h;
    const int gpr = a.hstride / 128;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int rr = c * 16 + lr;
      float amax = 0.f;
#pragma unroll
      for (int w = 0; w < kGateUpWaves; ++w) amax = fmaxf(amax, red[w * BM + rr]);
      const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
      if (rr < tr.rows) {
        const size_t row = (size_t)(hrow0 + rr);
        const uint32_t hv = pack4_e4m3(h[c][0] / sc, h[c][1] / sc, h[c][2] / sc, h[c][3] / sc);
        uint8_t* hp = hq + row * a.hstride + fcol;
        if constexpr (COH) {
          store_coherent(hp, hv);
          if (wave == 0 && lane < 16) store_coherent(&a.sh[row * gpr + nb], __float_as_uint(sc));
        } else {
          *(uint32_t*)hp = hv;
          if (wave == 0 && lane < 16) a.sh[row * gpr + nb] = sc;
        }
      }
    }
  } else {
    uint16_t* hb = (uint16_t*)a.h;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int rr = c * 16 + lr;
      if (rr < tr.rows) {
        const size_t row = (size_t)(hrow0 + rr);
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(h[c][0]) | ((uint32_t)f32_to_bf16(h[c][1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(h[c][2]) | ((uint32_t)f32_to_bf16(h[c][3]) << 16);
        uint16_t* hp = hb + row * a.hstride + fcol;
        if constexpr (COH) {
          store_coherent(hp, pk.x);
          store_coherent(hp + 2, pk.y);
        } else {
          *(uint2*)hp = pk;
        }
      }
    }
  }
  return true;
}

template <int BM, int WT, bool XB, bool A16 = false>
__global__ __launch_bounds__(kGateUpWaves * 64) void gateup_mfma_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  gateup_block<BM, WT, XB, false, A16>(a, blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// Down projection on the matrix cores; epilogue multiplies by the pair's
// routing weight (1 for the shared expert) and writes the fp32 partial row of
// pair p (or P + t).  A block of NW waves takes one tile and one slice of
// NW*16*RT output features (see block_rows); wave w owns RT 16-row tiles
// (features (nb*NW + w)*16*RT + 16 r).  RT = 2 for short tiles, RT = 4 for
// tall ones (a tile's h rows are staged once per 256 features); RT = 1 when a
// row's K does not fit one stage.
// ---------------------------------------------------------------------------
// A16 (with WT = 2): W8A16 -- h rows are bf16 with unit scales.
template <int BM, int WT, int RT, int NW, bool COH = false, bool A16 = false>
__device__ __forceinline__ void down_block(const ExpertArgs& a, int b, uint8_t* smem) {
  static_assert(!A16 || WT == 2, "W8A16 reads bf16 h rows for FP8 weights");
  constexpr bool HQ = WT == 2 && !A16;  // h as E4M3 codes with scales
  constexpr int NC = BM / 16;
  constexpr int EB = WT == 2 ? 1 : 2;   // bytes per weight element
  constexpr int EH = HQ ? 1 : 2;        // bytes per h element
  constexpr int KG = RT == 1 ? 10 : 5;  // K blocks requested per stage
  constexpr int NT = NW * 64;
  int nb;
  const TileRows tr = block_rows(a, b, nb);
  if (tr.g < 0) return;
  const int Fg = tr.shared ? a.Fs : a.F;
  const int RB = Fg * EB;          // bytes per W_down row
  const int nbb = RB / 128;
  const int hstride_b = a.hstride * EH;
  const int lstride = Fg * 2 + kLdsRowPad;  // padded LDS row: h as bf16
  uint8_t* hs = smem;
  float* shs = (float*)(smem + (BM + 1) * lstride);          // [Fg/128][BM] (FP8): one K block's rows adjacent
  float* wrow = shs + (WT == 2 ? BM * (Fg / 128) : 0);       // [BM] routing weight
  int* orow = (int*)(wrow + BM);                             // [BM] partial-output row
  float* wsd = (float*)(orow + BM);                          // [1 or 2][Fg/128] W_down block scales

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lk = (lane >> 4) * 16;
  const int n0 = (nb * NW + wave) * 16 * RT;
  const bool wave_live = n0 < a.d;  // d is a multiple of 16*RT here: whole waves are live or not
  const uint8_t* wd = tr.shared ? (const uint8_t*)a.shd : (const uint8_t*)a.wd + (size_t)tr.g * a.d * RB;
  const int nl = wave_live ? n0 : 0;
  const WeightStream ws = weight_stream(wd, RB, nl, a.w_tiled, lane, RT);
  // W_down block scales of the block's NW*16*RT rows (one or two 128-row scale
  // blocks), staged in LDS with h; the wave's row of them
  constexpr int nsr = NW * 16 * RT > 128 ? NW * 16 * RT / 128 : 1;
  static_assert(nsr <= 2, "LDS holds two rows of W_down scales");
  const int srow0 = nb * NW * 16 * RT / 128;
  const float* sdp = wsd + (nl / 128 - srow0) * (Fg / 128);
  // The weight stream depends only on the tile's expert and feature slice:
  // request it before the h rows are staged.  A stage = KG K blocks of one
  // 16-row tile; two stages in flight.
  v4i wlo[2][KG], whi[2][KG];
  auto load = [&](int slot, int r, int q0) {
#pragma unroll
    for (int j = 0; j < KG; ++j) {  // unconditional: past the row's end the last K block is read again
      const int so = r * ws.tile_step + min(q0 + j, nbb - 1) * ws.kb_stride;
      wlo[slot][j] = stream_load<WT == 2 && BM == 16>(ws, so);
      whi[slot][j] = stream_load<WT == 2 && BM == 16>(ws, so + ws.hi_off);
    }
  };
  // Staging, in pinned issue order (loads complete in issue order as far as
  // the wait counter goes): the pair rows, the h scales, the W_down scales and
  // the first batch of h rows, then the weight stream, then the routing
  // weights (which need the pair rows).  Unconditional loads from clamped
  // addresses and a spare LDS row for chunks past the tile: the code is
  // straight-line and every wait is exact.
  constexpr int SB = BM == 32 ? 5 : 4;  // one batch covers a 32-row tile of h codes at F = 640
  const int hrow0 = tr.hrow0, rlast = tr.rows - 1;
  const int cpr = Fg * EH / 16, nch = BM * cpr, nkb = Fg / 128, gpr = a.hstride / 128;
  const uint8_t* hsrc = (const uint8_t*)a.h;
  const int o = a.ri.prow[hrow0 + min(tid, rlast)];
  float sv = 0.f, dv = 0.f;
  if (WT == 2) {
    const float* shp = a.sh + (size_t)(hrow0 + min(tid % BM, rlast)) * gpr + min(tid / BM, nkb - 1);
    sv = !HQ ? 1.0f : COH ? __uint_as_float(load_coherent(shp)) : *shp;
    const float* sd = (tr.shared ? a.ssd : a.sd + (size_t)tr.g * (a.d / 128) * nkb) + (size_t)srow0 * nkb;
    dv = sd[min(tid, nsr * nkb - 1)];
  }
  // Chunk i is chunk i % cpr of row i / cpr.  A thread's batch is chunks
  // i0 + u*NT, whose row and chunk advance by NT / cpr and NT % cpr: one
  // division per batch rather than two per chunk.
  struct Batch {
    int r[SB], c[SB];
  };
  auto stage_walk = [&](int i0) {
    const int dr = NT / cpr, dc = NT - dr * cpr;
    int r = i0 / cpr, c = i0 - r * cpr;
    Batch bt;
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      bt.r[u] = r;
      bt.c[u] = c;
      r += dr;
      c += dc;
      const bool wrap = c >= cpr;
      r += wrap ? 1 : 0;
      c -= wrap ? cpr : 0;
    }
    return bt;
  };
  auto stage_load = [&](const Batch& bt, v4i (&v)[SB]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const uint8_t* hp = hsrc + (size_t)(hrow0 + min(bt.r[u], rlast)) * hstride_b + bt.c[u] * 16;
      if constexpr (COH) {  // coherent loads skip the L2: fetch only chunks of live rows
        v[u] = v4i{0, 0, 0, 0};
        if (bt.r[u] <= rlast)
          v[u] = v4i{(int)load_coherent(hp), (int)load_coherent(hp + 4), (int)load_coherent(hp + 8),
                     (int)load_coherent(hp + 12)};
      } else {
        v[u] = *(const v4i*)hp;
      }
    }
  };
  // Rows past the tile (r > rlast) hold copies of the last row (clamped loads;
  // zeros in the coherent path): their products are never stored.  Chunks
  // past the tile's last row (r >= BM) go to the spare row.
  auto stage_store = [&](const Batch& bt, const v4i (&v)[SB]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const bool in = bt.r[u] < BM;
      uint8_t* dst = hs + (in ? bt.r[u] : BM) * lstride;
      const int c = in ? bt.c[u] : 0;
      if constexpr (HQ) {  // E4M3 codes -> bf16 once per block (exact)
        v4i lo, hi;
        e4m3x16_to_bf16(v[u], lo, hi);
        *(v4i*)(dst + xunit_pos(c)) = lo;
        *(v4i*)(dst + xunit_pos(c) + 64) = hi;
      } else if constexpr (WT == 2) {  // bf16 h (W8A16): 8 elements of a unit
        *(v4i*)(dst + xunit_pos(c >> 1) + 64 * (c & 1)) = v[u];
      } else {
        *(v4i*)(dst + c * 16) = v[u];
      }
    }
  };
  v4i hv[SB];
  const Batch bt0 = stage_walk(tid);
  stage_load(bt0, hv);
  __builtin_amdgcn_sched_barrier(0);
  load(0, 0, 0);
  if (RT > 1) load(1, 1, 0);
  __builtin_amdgcn_sched_barrier(0);
  const float wt = a.ri.w[hrow0 + min(tid, rlast)];
  stage_store(bt0, hv);
  for (int i0 = tid + NT * SB; i0 < nch; i0 += NT * SB) {  // tall tiles or wide rows only
    const Batch bt = stage_walk(i0);
    stage_load(bt, hv);
    stage_store(bt, hv);
  }
  if (WT == 2) {
    if (tid < BM * nkb) shs[tid] = tid % BM <= rlast ? sv : 0.f;
    for (int i = tid + NT; i < BM * nkb; i += NT) {  // tall tiles or wide rows only
      const float* shp = a.sh + (size_t)(hrow0 + min(i % BM, rlast)) * gpr + i / BM;
      shs[i] = i % BM <= rlast ? (!HQ ? 1.0f : COH ? __uint_as_float(load_coherent(shp)) : *shp) : 0.f;
    }
    if (tid < nsr * nkb) wsd[tid] = dv;
  }
  if (tid < BM) {
    orow[tid] = tid <= rlast ? o : -1;
    wrow[tid] = tid <= rlast ? wt : 0.f;
  }
  __syncthreads();
  if (!wave_live) return;

  v4f acc[RT][NC];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int slot, int r, int q0) {
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const int bb = q0 + j;
      if (bb >= nbb) break;
      v4i wd[4];  // the K block's weight codes decoded once for every row chunk
      if constexpr (WT == 2) kblock_decode(wlo[slot][j], whi[slot][j], wd);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (WT == 2) {
          const uint8_t* bp = hs + (c * 16 + lr) * lstride + bb * 256 + lk;  // xunit_pos layout
          const v4i b[4] = {*(const v4i*)bp, *(const v4i*)(bp + 64), *(const v4i*)(bp + 128),
                            *(const v4i*)(bp + 192)};
          // the wave's 16*RT <= 64 rows start at a multiple of 64: one 128-row scale block
          acc[r][c] += kblock_bf16(wd, b) * (shs[bb * BM + c * 16 + lr] * sdp[bb]);
        } else {
          const uint8_t* bp = hs + (c * 16 + lr) * lstride + bb * 128 + lk;
          const v4i blo = *(const v4i*)bp;
          const v4i bhi = *(const v4i*)(bp + 64);
          acc[r][c] = mfma_bf16(wlo[slot][j], blo, acc[r][c]);
          acc[r][c] = mfma_bf16(whi[slot][j], bhi, acc[r][c]);
        }
      }
    }
  };
  if constexpr (RT == 1) {
    // short rows: one tile, groups of KG K blocks
    compute(0, 0, 0);
    for (int q0 = KG; q0 < nbb; q0 += KG) {
      load(0, 0, q0);
      compute(0, 0, q0);
    }
  } else {
    // RT tiles of up to KG K blocks each (nbb <= KG), two in flight
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      compute(r & 1, r, 0);
      if (r + 2 < RT) load(r & 1, r + 2, 0);
    }
  }

#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int rr = c * 16 + lr;
      if (rr < tr.rows) {
        const v4f v = acc[r][c] * wrow[rr];
        *(float4*)(a.part + (size_t)orow[rr] * a.d + n0 + r * 16 + 4 * (lane >> 4)) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
    }
}

// (256, 2): at most 256 registers per lane, so the products accumulate in
// vector registers rather than in accumulation registers read back one by one.
template <int BM, int WT, int RT, bool A16 = false>
__global__ __launch_bounds__(256, 2) void down_mfma_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  down_block<BM, WT, RT, 4, false, A16>(a, blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// 4-bit weights (MOE_U4_G64): element value = scale * q + bias per (row, group
// of 64 columns), bf16 activations and h.  The codes arrive in
// MOE_LAYOUT_TILED as moe_pack_weights_u4 writes them: per 16-row tile and
// 128-column block 1 KB, in which lane l's 16 bytes (at 16*l) belong to row
// l%16 and word m of them to columns 128*kb + 32*m + 8*(l/16) + [0, 8), nibble
// order (0, 2, 4, 6 | 1, 3, 5, 7), so that (w >> 4i) & 0x000F000F isolates
// columns 2i and 2i+1 in the two 16-bit halves.  OR-ing 0x4300 into a half
// makes it the bf16 value 128 + q exactly, and the matrix cores sum
// x * (128 + q) exactly-multiplied in fp32 over each 32-column step.  A group
// is two whole steps, so per group
//     sum_i x_i * (scale * q_i + bias) = scale * S + (bias - 128 * scale) * X
// with S the group's matrix-core sum and X = sum_i x_i (added up once per row
// while the rows are staged).  The weights are the B operand: a lane's output
// column is its own weight row, so it needs one (scale, bias) pair per group,
// and the packed group parameters give it 8 bytes per 128-column block (the
// scale and bias of its row's two groups).  Output lanes hold rows 4*(l/16) + v
// of one column; a 4x4 transpose inside each quad of lanes turns that into four
// consecutive columns of one row for the stores.
// ---------------------------------------------------------------------------

// Eight 4-bit codes (one packed word) as eight bf16 values 128 + q.  The two
// constants are passed in registers (made opaque to the compiler) so that each
// half-word pair costs one shift and one and-or instead of a shift, an and and
// an or with literal operands.
struct U4Consts {
  uint32_t mask, high;
};
__device__ __forceinline__ U4Consts u4_consts() {
  U4Consts k{0x000F000Fu, 0x43004300u};
  asm volatile("" : "+s"(k.mask));
  asm volatile("" : "+v"(k.high));
  return k;
}
__device__ __forceinline__ v4i u4_word_to_bf16(uint32_t w, U4Consts k) {
  v4i r;
  r[0] = (int)((w & k.mask) | k.high);
  r[1] = (int)(((w >> 4) & k.mask) | k.high);
  r[2] = (int)(((w >> 8) & k.mask) | k.high);
  r[3] = (int)(((w >> 12) & k.mask) | k.high);
  return r;
}

// Sum of the eight bf16 values of a 16-byte chunk, then over the eight
// consecutive lanes that hold one 64-column group (all lanes must call it).
__device__ __forceinline__ float group_sum_bf16x8(v4i x) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    s += __uint_as_float((uint32_t)x[j] << 16) + __uint_as_float((uint32_t)x[j] & 0xffff0000u);
  s += __shfl_xor(s, 1, kWave);
  s += __shfl_xor(s, 2, kWave);
  s += __shfl_xor(s, 4, kWave);
  return s;
}

// acc plus one 64-column group's contribution to a lane's four outputs: S is
// the matrix-core sum of x * (128 + q), pv the group's bf16 scale (low half)
// and bias (high half), X the four rows' sums of x over the group.
__device__ __forceinline__ v4f u4_group_add(v4f acc, v4f S, uint32_t pv, v4f X) {
  const float sc = __uint_as_float(pv << 16), bi = __uint_as_float(pv & 0xffff0000u);
  const float b128 = fmaf(-128.0f, sc, bi);
#pragma unroll
  for (int v = 0; v < 4; ++v) acc[v] = fmaf(sc, S[v], fmaf(b128, X[v], acc[v]));
  return acc;
}

// 4x4 transpose inside each quad of lanes: lane i of a quad holds column i of
// a 4x4 block (a[v] = C[v][i]); afterwards it holds row i (a[v] = C[i][v]).
// All lanes must call it.
__device__ __forceinline__ v4f quad_transpose(v4f a) {
  const int i = threadIdx.x & 3;
  const bool odd = i & 1, upper = i & 2;
  float s0 = odd ? a[0] : a[1], s1 = odd ? a[2] : a[3];
  float r0 = __shfl_xor(s0, 1, kWave), r1 = __shfl_xor(s1, 1, kWave);
  if (odd) {
    a[0] = r0;
    a[2] = r1;
  } else {
    a[1] = r0;
    a[3] = r1;
  }
  s0 = upper ? a[0] : a[2];
  s1 = upper ? a[1] : a[3];
  r0 = __shfl_xor(s0, 2, kWave);
  r1 = __shfl_xor(s1, 2, kWave);
  if (upper) {
    a[0] = r0;
    a[1] = r1;
  } else {
    a[2] = r0;
    a[3] = r1;
  }
  return a;
}

// Gate/up with 4-bit weights: 16-row tiles, 8 waves, one 128-feature group nb
// of h per block (as for FP8 weights); wave w owns features nb*128 + 16w +
// [0, 16) of W_gate and W_up.  A stage is KG blocks of 128 columns of both
// matrices (gate blocks, then the same up blocks), two stages in flight, so
// that each activation chunk and group sum read from LDS serves both.  COH: h
// stored coherently (the fused expert launch).
#ifndef MOE_U4_KG
#define MOE_U4_KG 2  // 128-column blocks of each matrix per stage
#endif
template <bool COH>
__device__ __forceinline__ bool gateup_block_u4(const ExpertArgs& a, int b, uint8_t* smem) {
  constexpr int BM = 16, NT = kGateUpWaves * 64, KG = MOE_U4_KG, SB = 4;
  int nb;
  const TileRows tr = block_rows(a, b, nb);
  if (tr.g < 0) return false;
  const int Fg = tr.shared ? a.Fs : a.F;
  if (nb * 128 >= Fg) return false;
  const int d = a.d, nkb = d / 128, ng = d / 64;
  const int xstride = d * 2 + kLdsRowPad;             // padded LDS row of bf16 activations
  uint8_t* xs = smem;                                 // [BM + 1][xstride] (a spare row)
  float* xsum = (float*)(smem + (BM + 1) * xstride);  // [d/64][BM] group sums of each row

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, q4 = lane >> 4;
  const size_t cbytes = (size_t)a.F * d / 2, pbytes = (size_t)a.F * ng * 4;  // one routed matrix
  const uint8_t* cg = tr.shared ? (const uint8_t*)a.shg : (const uint8_t*)a.wg + (size_t)tr.g * cbytes;
  const uint8_t* cu = tr.shared ? (const uint8_t*)a.shu : (const uint8_t*)a.wu + (size_t)tr.g * cbytes;
  const uint8_t* pg = tr.shared ? (const uint8_t*)a.ssg : (const uint8_t*)a.sg + (size_t)tr.g * pbytes;
  const uint8_t* pu = tr.shared ? (const uint8_t*)a.ssu : (const uint8_t*)a.su + (size_t)tr.g * pbytes;
  const int f0 = nb * 128 + wave * 16;
  const size_t t0 = (size_t)(f0 / 16) * nkb;  // the wave's first tile block
  // the wave's tile of each matrix: codes (1 KB per block) and parameters (128 B)
  const __amdgpu_buffer_rsrc_t rc[2] = {buffer_over(cg + t0 * 1024, nkb * 1024), buffer_over(cu + t0 * 1024, nkb * 1024)};
  const __amdgpu_buffer_rsrc_t rp[2] = {buffer_over(pg + t0 * 128, nkb * 128), buffer_over(pu + t0 * 128, nkb * 128)};

  // Stage q: blocks [q*KG, q*KG + KG) of W_gate, then of W_up.  Loads are
  // unconditional (a short last stage re-reads the final block, in bounds).
  const int ns = (nkb + KG - 1) / KG;
  v4i wc[2][2][KG];
  uint2 wp[2][2][KG];
  auto load = [&](auto S, int q) {
    constexpr int sl = decltype(S)::value;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < KG; ++j) {
        const int kb = min(q * KG + j, nkb - 1);
        wc[sl][m][j] = buffer_load16<true>(rc[m], lane * 16, kb * 1024);
        wp[sl][m][j] = buffer_load8(rp[m], lr * 8, kb * 128);
      }
  };

  // Staging, in pinned issue order: row tokens, the weight stream, then the
  // activation rows (bf16) and their per-group sums.  Only the tile's live
  // rows are staged: rows past them keep whatever the LDS held, and feed only
  // output rows that are never stored (each output row of a product reads its
  // own activation row and group sums alone).
  const int cpr = d / 8, nch = tr.rows * cpr;  // 16-byte chunks per row / of the live rows
  const uint8_t* xa = (const uint8_t*)a.xa;
  const int rlast = tr.rows - 1;
  // Chunk i is chunk i % cpr of row i / cpr; a thread's chunks i0 + u*NT
  // advance by NT / cpr rows and NT % cpr chunks (one division per batch).
  // A batch runs only the chunk slots some thread needs (a uniform count);
  // chunks past the live rows re-read the last row and go to the spare row.
  auto stage = [&](int i0, bool first) {
    const int slots = min(SB, (nch - (i0 - tid) + NT - 1) / NT);  // >= 1
    int rs[SB], cs[SB];
    {
      const int dr = NT / cpr, dc = NT - dr * cpr;
      int r = i0 / cpr, c = i0 - r * cpr;
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        rs[u] = r;
        cs[u] = c;
        r += dr;
        c += dc;
        const bool wrap = c >= cpr;
        r += wrap ? 1 : 0;
        c -= wrap ? cpr : 0;
      }
    }
    int tk[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u)
      if (u < slots) tk[u] = a.ri.tok[tr.hrow0 + min(rs[u], rlast)];
    if (first) {
      __builtin_amdgcn_sched_barrier(0);
      load(Ic<0>{}, 0);
      load(Ic<1>{}, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    v4i v[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u)
      if (u < slots) v[u] = *(const v4i*)(xa + (size_t)tk[u] * d * 2 + cs[u] * 16);
#pragma unroll
    for (int u = 0; u < SB; ++u)
      if (u < slots) {
        const bool in = rs[u] <= rlast;
        *(v4i*)(xs + (in ? rs[u] : BM) * xstride + (in ? cs[u] : 0) * 16) = v[u];
        const float s = group_sum_bf16x8(v[u]);  // the group's 8 chunks sit in 8 consecutive lanes
        if ((tid & 7) == 0 && in) xsum[(cs[u] / 8) * BM + rs[u]] = s;
      }
  };
  stage(tid, true);
  for (int i0 = tid + NT * SB; i0 - tid < nch; i0 += NT * SB) stage(i0, false);
  __syncthreads();

  v4f acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const U4Consts kc = u4_consts();
  auto compute = [&](auto S, int q) {
    constexpr int sl = decltype(S)::value;
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const int kb = q * KG + j;
      if (kb >= nkb) break;
      const uint8_t* xp = xs + lr * xstride + kb * 256 + q4 * 16;  // columns 128 kb + 32 m + 8 q4
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4i x0 = *(const v4i*)(xp + 128 * h), x1 = *(const v4i*)(xp + 128 * h + 64);
        const v4f X = *(const v4f*)(xsum + (2 * kb + h) * BM + 4 * q4);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          v4f S = {0.f, 0.f, 0.f, 0.f};
          S = mfma_bf16(x0, u4_word_to_bf16((uint32_t)wc[sl][m][j][2 * h], kc), S);
          S = mfma_bf16(x1, u4_word_to_bf16((uint32_t)wc[sl][m][j][2 * h + 1], kc), S);
          acc[m] = u4_group_add(acc[m], S, h ? wp[sl][m][j].y : wp[sl][m][j].x, X);
        }
      }
    }
  };
  int q = 0;
  for (; q + 2 < ns; q += 2) {
    compute(Ic<0>{}, q);
    load(Ic<0>{}, q + 2);
    compute(Ic<1>{}, q + 1);
    load(Ic<1>{}, q + 3);
  }
  compute(Ic<0>{}, q);
  if (q + 1 < ns) compute(Ic<1>{}, q + 1);

  // h = silu(g) * u for rows 4*q4 + v of feature f0 + lr, then transposed to
  // row 4*q4 + lane%4, features f0 + 4*((lane/4)%4) + v.
  v4f hv;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float gv = acc[0][v], uv = acc[1][v];
    hv[v] = silu_f32(gv) * uv;
  }
  hv = quad_transpose(hv);
  const int rr = 4 * q4 + (lane & 3);
  if (rr < tr.rows) {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(hv[0]) | ((uint32_t)f32_to_bf16(hv[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16(hv[2]) | ((uint32_t)f32_to_bf16(hv[3]) << 16);
    uint16_t* hp = (uint16_t*)a.h + (size_t)(tr.hrow0 + rr) * a.hstride + f0 + 4 * ((lane >> 2) & 3);
    if constexpr (COH) {
      store_coherent(hp, pk.x);
      store_coherent(hp + 2, pk.y);
    } else {
      *(uint2*)hp = pk;
    }
  }
  return true;
}

template <bool COH>
__global__ __launch_bounds__(kGateUpWaves * 64) void gateup_u4_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  gateup_block_u4<COH>(a, blockIdx.x, smem);
}

// Down projection with 4-bit weights: NW waves, each owning RT 16-row tiles
// of W_down (features (nb*NW + w)*16*RT + 16 r).  RT = 2 holds both tiles'
// whole rows in registers (F <= 640: up to 5 blocks of 128 columns each);
// RT = 1 streams one tile's row in stages of 4 blocks, two in flight.  The
// epilogue multiplies by the pair's routing weight and writes fp32 partials.
template <int RT, int NW, bool COH>
__device__ __forceinline__ void down_block_u4(const ExpertArgs& a, int b, uint8_t* smem) {
  constexpr int BM = 16, NT = NW * 64, SB = 4;
  constexpr int KG = RT == 2 ? 5 : 4;  // 128-column blocks per register slot
  int nb;
  const TileRows tr = block_rows(a, b, nb);
  if (tr.g < 0) return;
  const int Fg = tr.shared ? a.Fs : a.F;
  const int nkb = Fg / 128, ng = Fg / 64;
  const int lstride = Fg * 2 + kLdsRowPad;
  uint8_t* hs = smem;                                 // [BM + 1][lstride] bf16 h rows
  float* hsum = (float*)(smem + (BM + 1) * lstride);  // [Fg/64][BM] group sums of each row
  float* wrow = hsum + ng * BM;                       // [BM] routing weight
  int* orow = (int*)(wrow + BM);                      // [BM] partial-output row

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, q4 = lane >> 4;
  const int n0 = (nb * NW + wave) * 16 * RT;
  const bool wave_live = n0 < a.d;  // d is a multiple of 16*RT: whole waves are live or not
  const int nl = wave_live ? n0 : 0;
  const size_t cbytes = (size_t)a.d * a.F / 2, pbytes = (size_t)a.d * (a.F / 64) * 4;  // one routed matrix
  const uint8_t* cd = tr.shared ? (const uint8_t*)a.shd : (const uint8_t*)a.wd + (size_t)tr.g * cbytes;
  const uint8_t* pd = tr.shared ? (const uint8_t*)a.ssd : (const uint8_t*)a.sd + (size_t)tr.g * pbytes;
  const size_t t0 = (size_t)(nl / 16) * nkb;
  // the wave's RT tiles (tile r: + r * nkb blocks): codes and parameters
  const __amdgpu_buffer_rsrc_t rc = buffer_over(cd + t0 * 1024, RT * nkb * 1024);
  const __amdgpu_buffer_rsrc_t rp = buffer_over(pd + t0 * 128, RT * nkb * 128);

  v4i wc[2][KG];
  uint2 wp[2][KG];
  auto load = [&](auto S, int r, int q) {  // blocks [q*KG, q*KG + KG) of tile r (clamped: re-reads in bounds)
    constexpr int sl = decltype(S)::value;
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const int kb = r * nkb + min(q * KG + j, nkb - 1);
      wc[sl][j] = buffer_load16<true>(rc, lane * 16, kb * 1024);
      wp[sl][j] = buffer_load8(rp, lr * 8, kb * 128);
    }
  };

  // Staging, in pinned issue order: h rows, the weight stream, the rows'
  // routing weights and output rows; then h to LDS with its group sums.
  const int hrow0 = tr.hrow0, rlast = tr.rows - 1;
  const int cpr = Fg / 8, nch = tr.rows * cpr;  // chunks of the live rows
  const uint8_t* hsrc = (const uint8_t*)a.h;
  const int o = a.ri.prow[hrow0 + min(tid, rlast)];
  // Chunk i is chunk i % cpr of row i / cpr; a thread's chunks i0 + u*NT
  // advance by NT / cpr rows and NT % cpr chunks (one division per batch).
  struct Batch {
    int r[SB], c[SB], slots;
  };
  // A batch runs only the chunk slots some thread needs (a uniform count).
  auto stage_walk = [&](int i0) {
    const int dr = NT / cpr, dc = NT - dr * cpr;
    int r = i0 / cpr, c = i0 - r * cpr;
    Batch bt;
    bt.slots = min(SB, (nch - (i0 - tid) + NT - 1) / NT);  // >= 1
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      bt.r[u] = r;
      bt.c[u] = c;
      r += dr;
      c += dc;
      const bool wrap = c >= cpr;
      r += wrap ? 1 : 0;
      c -= wrap ? cpr : 0;
    }
    return bt;
  };
  auto stage_load = [&](const Batch& bt, v4i (&v)[SB]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      if (u >= bt.slots) continue;
      const uint8_t* hp = hsrc + ((size_t)(hrow0 + min(bt.r[u], rlast)) * a.hstride + bt.c[u] * 8) * 2;
      if constexpr (COH) {  // coherent loads skip the L2: fetch only chunks of live rows
        v[u] = v4i{0, 0, 0, 0};
        if (bt.r[u] <= rlast)
          v[u] = v4i{(int)load_coherent(hp), (int)load_coherent(hp + 4), (int)load_coherent(hp + 8),
                     (int)load_coherent(hp + 12)};
      } else {
        v[u] = *(const v4i*)hp;
      }
    }
  };
  // Only the live rows are staged: rows past them keep whatever the LDS held
  // and feed only output rows that are never stored.  Chunks past the live
  // rows (a re-read of the last row, or zeros in the coherent path) go to the
  // spare row.
  auto stage_store = [&](const Batch& bt, const v4i (&v)[SB]) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      if (u >= bt.slots) continue;
      const bool in = bt.r[u] <= rlast;
      *(v4i*)(hs + (in ? bt.r[u] : BM) * lstride + (in ? bt.c[u] : 0) * 16) = v[u];
      const float s = group_sum_bf16x8(v[u]);
      if ((tid & 7) == 0 && in) hsum[(bt.c[u] / 8) * BM + bt.r[u]] = s;
    }
  };
  v4i hv[SB];
  const Batch bt0 = stage_walk(tid);
  stage_load(bt0, hv);
  __builtin_amdgcn_sched_barrier(0);
  load(Ic<0>{}, 0, 0);
  if (RT == 2) load(Ic<1>{}, 1, 0);
  else load(Ic<1>{}, 0, 1);
  __builtin_amdgcn_sched_barrier(0);
  const float wt = a.ri.w[hrow0 + min(tid, rlast)];
  stage_store(bt0, hv);
  for (int i0 = tid + NT * SB; i0 - tid < nch; i0 += NT * SB) {
    const Batch bt = stage_walk(i0);
    stage_load(bt, hv);
    stage_store(bt, hv);
  }
  if (tid < BM) {
    orow[tid] = tid <= rlast ? o : -1;
    wrow[tid] = tid <= rlast ? wt : 0.f;
  }
  __syncthreads();
  if (!wave_live) return;

  v4f acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) acc[r] = v4f{0.f, 0.f, 0.f, 0.f};
  const U4Consts kc = u4_consts();
  auto compute = [&](auto R, auto S, int q) {
    constexpr int r = decltype(R)::value, sl = decltype(S)::value;
#pragma unroll
    for (int j = 0; j < KG; ++j) {
      const int kb = q * KG + j;
      if (kb >= nkb) break;
      const uint8_t* xp = hs + lr * lstride + kb * 256 + q4 * 16;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4f S = {0.f, 0.f, 0.f, 0.f};
        S = mfma_bf16(*(const v4i*)(xp + 128 * h), u4_word_to_bf16((uint32_t)wc[sl][j][2 * h], kc), S);
        S = mfma_bf16(*(const v4i*)(xp + 128 * h + 64), u4_word_to_bf16((uint32_t)wc[sl][j][2 * h + 1], kc), S);
        const v4f X = *(const v4f*)(hsum + (2 * kb + h) * BM + 4 * q4);
        acc[r] = u4_group_add(acc[r], S, h ? wp[sl][j].y : wp[sl][j].x, X);
      }
    }
  };
  if constexpr (RT == 2) {  // whole rows in registers (nkb <= KG)
    compute(Ic<0>{}, Ic<0>{}, 0);
    compute(Ic<1>{}, Ic<1>{}, 0);
  } else {
    const int nq = (nkb + KG - 1) / KG;
    int q = 0;
    for (; q + 2 < nq; q += 2) {
      compute(Ic<0>{}, Ic<0>{}, q);
      load(Ic<0>{}, 0, q + 2);
      compute(Ic<0>{}, Ic<1>{}, q + 1);
      load(Ic<1>{}, 0, q + 3);
    }
    compute(Ic<0>{}, Ic<0>{}, q);
    if (q + 1 < nq) compute(Ic<0>{}, Ic<1>{}, q + 1);
  }

  const int rr = 4 * q4 + (lane & 3);
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const v4f v = quad_transpose(acc[r]) * wrow[rr];
    if (rr < tr.rows)
      *(float4*)(a.part + (size_t)orow[rr] * a.d + n0 + r * 16 + 4 * ((lane >> 2) & 3)) =
          make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <int RT>
__global__ __launch_bounds__(256, 2) void down_u4_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  down_block_u4<RT, 4, false>(a, blockIdx.x, smem);
}

// ---------------------------------------------------------------------------
// Gate/up and down in one launch (FP8 weights with E4M3 or bf16 activations,
// or 4-bit weights; 16-row tiles, tile-list schedule).  Blocks [0, n_gu) do the
// gate/up work; the rest are 8-wave down blocks (256 output features each).  A
// gate/up block stores its h rows (and their scales) coherently (agent-scope atomic stores, written through to where every
// XCD reads them), waits until each of its waves' stores has completed, and
// then counts itself in ready[tile]; a down block of that tile waits until the
// count reaches the tile's gate/up slices and reads h and its scales with
// coherent loads issued after that.  No cache-wide writeback or invalidation
// is needed: device-scope fences (one L2 writeback or invalidation per block)
// cost more than the launch gap they remove.  The down blocks start while the
// last gate/up blocks are still streaming, which fills the launch's last,
// partly empty round of blocks, and the kernel boundary between the two
// projections disappears.
//
// Forward progress: blocks are dispatched in block order, so every gate/up
// block a down block waits for was dispatched before it, holds its own slot
// and never waits itself.  The wait is bounded all the same: past kSpinLimit
// polls the block sets the routing status word to MOE_ERR_DEVICE_SYNC and goes
// on (its output is then not valid).  The routing call zeroes ready[] and
// done[] with the plan; the last down block of a tile zeroes them again, so the
// plan can serve any number of forward calls (one at a time).
// ---------------------------------------------------------------------------
constexpr int kSpinLimit = 1 << 22;  // polls of about 64 cycles each: far beyond any real wait

// WM: the weight mode -- 2 FP8, 3 FP8 as W8A16, 4 4-bit groups.
// need_extra / spin_limit: 0 and kSpinLimit, except in the error-path test (1 and 16).
template <int WM>
__global__ __launch_bounds__(kGateUpWaves * 64) void experts_fused_kernel(ExpertArgs gu, ExpertArgs dn, int n_gu,
                                                                          int32_t* __restrict__ ready,
                                                                          int32_t* __restrict__ done,
                                                                          int32_t* __restrict__ status,
                                                                          int32_t* __restrict__ sticky,
                                                                          int need_extra, int spin_limit) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int b = blockIdx.x;
  if (b < n_gu) {
    bool worked;
    if constexpr (WM == 4) worked = gateup_block_u4<true>(gu, b, smem);
    else worked = gateup_block<16, 2, true, true, WM == 3>(gu, b, smem);
    if (worked) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's coherent stores have completed ...
      __syncthreads();                // ... and so have every other wave's
      if (threadIdx.x == 0) atomicAdd(&ready[b / gu.nsl], 1);
    }
    return;
  }
  const int bd = b - n_gu, tile = bd / dn.nsl;
  const int4 rec = dn.sched[tile];
  if (rec.x < 0) return;
  const int need = (rec.x == dn.E ? dn.Fs : dn.F) / 128 + need_extra;  // gate/up slices of the tile
  if (threadIdx.x == 0) {
    int polls = 0;
    while (__hip_atomic_load(&ready[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
      __builtin_amdgcn_s_sleep(1);
      if (++polls >= spin_limit) {
        *status = MOE_ERR_DEVICE_SYNC;
        if (sticky) *sticky = MOE_ERR_DEVICE_SYNC;
        break;
      }
    }
  }
  __syncthreads();  // h is read below, with coherent loads, after the count was seen
  if constexpr (WM == 4) down_block_u4<2, kGateUpWaves, true>(dn, bd, smem);
  else down_block<16, 2, 2, kGateUpWaves, true, WM == 3>(dn, bd, smem);
  __syncthreads();
  if (threadIdx.x == 0 && atomicAdd(&done[tile], 1) == dn.nsl - 1) {  // the tile's last down block
    atomicExch(&ready[tile], 0);
    atomicExch(&done[tile], 0);
  }
}

// ---------------------------------------------------------------------------
// fp32 expert projections (fp32 activations and weights): plain fp32
// multiply-add, one output feature per thread, each sum a single chain over
// the input columns in order.  blockIdx.x = 64-feature slice.  The inputs go
// through LDS in chunks of kF32Chunk columns: the tile's rows (zeros past the
// live rows) and the slice's 64 weight rows, read with 16-byte loads where 16
// threads cover a row's chunk; weight rows padded to kF32Chunk + 1 floats so
// that 64 lanes reading one column of 64 rows hit distinct banks.  Thread
// (feature f, row group g) takes rows g, g + 4, g + 8, g + 12.
// ---------------------------------------------------------------------------
constexpr int kF32Chunk = 64;

template <int BM>
__global__ __launch_bounds__(256) void gateup_f32_kernel(ExpertArgs a) {
  static_assert(BM == 16, "four rows per thread");
  int sl;
  const TileRows tr = block_rows(a, blockIdx.x, sl);
  if (tr.g < 0) return;
  const int Fg = tr.shared ? a.Fs : a.F;
  if (sl * 64 >= Fg) return;
  __shared__ __align__(16) float xs[BM][kF32Chunk];
  __shared__ float gs[64][kF32Chunk + 1], us[64][kF32Chunk + 1];
  const int tid = threadIdx.x, fl = tid & 63, rg = tid >> 6, f = sl * 64 + fl;
  const float* x = (const float*)a.xa;
  const size_t wsz = (size_t)a.F * a.d;
  const float* wg = tr.shared ? (const float*)a.shg : (const float*)a.wg + tr.g * wsz;
  const float* wu = tr.shared ? (const float*)a.shu : (const float*)a.wu + tr.g * wsz;
  // this thread's staging slots: x row tid / 16 (one per thread), weight rows
  // tid / 16 + 16 j, each 4 floats at column 4 * (tid % 16)
  const int sr = tid >> 4, sc = 4 * (tid & 15);
  int tok = -1;
  if (sr < tr.rows) tok = tr.shared ? tr.m0 + sr : a.perm[tr.hrow0 + sr] / a.k;
  float g[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.d; k0 += kF32Chunk) {
    __syncthreads();  // the previous chunk's reads are done
    *(float4*)&xs[sr][sc] = tok >= 0 ? *(const float4*)(x + (size_t)tok * a.d + k0 + sc) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int fr = min(sl * 64 + sr + 16 * j, Fg - 1);  // rows past the matrix: a clamped copy, never stored
      const float4 vg = *(const float4*)(wg + (size_t)fr * a.d + k0 + sc);
      const float4 vu = *(const float4*)(wu + (size_t)fr * a.d + k0 + sc);
      float* dg = &gs[sr + 16 * j][sc];
      float* du = &us[sr + 16 * j][sc];
      dg[0] = vg.x; dg[1] = vg.y; dg[2] = vg.z; dg[3] = vg.w;
      du[0] = vu.x; du[1] = vu.y; du[2] = vu.z; du[3] = vu.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kF32Chunk; ++c) {
      const float wgv = gs[fl][c], wuv = us[fl][c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g[i] = fmaf(wgv, xs[rg + 4 * i][c], g[i]);
        u[i] = fmaf(wuv, xs[rg + 4 * i][c], u[i]);
      }
    }
  }
  if (f >= Fg) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rg + 4 * i;
    if (r < tr.rows) ((float*)a.h)[(size_t)(tr.hrow0 + r) * a.hstride + f] = g[i] / (1.0f + expf(-g[i])) * u[i];
  }
}

template <int BM>
__global__ __launch_bounds__(256) void down_f32_kernel(ExpertArgs a) {
  static_assert(BM == 16, "four rows per thread");
  int sl;
  const TileRows tr = block_rows(a, blockIdx.x, sl);
  if (tr.g < 0) return;
  const int Fg = tr.shared ? a.Fs : a.F;
  if (sl * 64 >= a.d) return;
  __shared__ __align__(16) float hs[BM][kF32Chunk];
  __shared__ float ws[64][kF32Chunk + 1];
  const int tid = threadIdx.x, nl = tid & 63, rg = tid >> 6, n = sl * 64 + nl;
  const float* wd = tr.shared ? (const float*)a.shd : (const float*)a.wd + tr.g * (size_t)a.d * Fg;
  const int sr = tid >> 4, sc = 4 * (tid & 15);
  const float* hrow = sr < tr.rows ? (const float*)a.h + (size_t)(tr.hrow0 + sr) * a.hstride : nullptr;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < Fg; k0 += kF32Chunk) {
    __syncthreads();
    *(float4*)&hs[sr][sc] = hrow ? *(const float4*)(hrow + k0 + sc) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int nr = min(sl * 64 + sr + 16 * j, a.d - 1);
      const float4 v = *(const float4*)(wd + (size_t)nr * Fg + k0 + sc);
      float* dst = &ws[sr + 16 * j][sc];
      dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < kF32Chunk; ++c) {
      const float w = ws[nl][c];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, hs[rg + 4 * i][c], acc[i]);
    }
  }
  if (n >= a.d) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = rg + 4 * i;
    if (r >= tr.rows) continue;
    int o;
    float w;
    if (tr.shared) {
      o = a.P + tr.m0 + r;
      w = 1.f;
    } else {
      o = a.perm[tr.hrow0 + r];
      w = a.topk_w[o];
    }
    a.part[(size_t)o * a.d + n] = acc[i] * w;
  }
}

// ---------------------------------------------------------------------------
// Combine, fixed order per token: acc = shared; acc += (w_j * y_j) for
// j = 0..k-1 (the products were formed in the down epilogue); y = round(acc).
// Invalid slots (id -1) are skipped.  Eight features per thread (d is a
// multiple of 128).  NT: the partials are read with the streaming hint, for
// partial buffers larger than the chip's 256 MB last-level cache (measured on
// MI355X: -12 us at T = 8192, +2 us at T = 2048, whose 117 MB of partials the
// cache still holds from the down launch).
// ---------------------------------------------------------------------------
template <bool BF16OUT, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part,
                                                      const int32_t* __restrict__ idx, int T, int k, int d, int E,
                                                      int P, int has_shared, void* __restrict__ y) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = d / 8;
  if (gid >= (int64_t)T * q) return;
  const int t = (int)(gid / q), n = (int)(gid - (int64_t)t * q) * 8;
  // every slot's row is requested together with the ids (the rows of invalid
  // slots are in bounds and skipped), so the call costs one round trip
  auto ld = [&](size_t row, float (&v)[8]) {
    const v4f* p = (const v4f*)(part + row * d + n);
    v4f a, b;
    if constexpr (NT) {
      a = __builtin_nontemporal_load(p);
      b = __builtin_nontemporal_load(p + 1);
    } else {
      a = p[0];
      b = p[1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  };
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (has_shared) ld((size_t)P + t, acc);
  float v[kMaxTopK][8];
  int ev[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) {
      ev[j] = idx[(size_t)t * k + j];
      ld((size_t)t * k + j, v[j]);
    }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k || ev[j] < 0 || ev[j] >= E) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] + v[j][i];
  }
  if (BF16OUT) {
    uint4 pk;
    pk.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    pk.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    pk.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    pk.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    *(uint4*)((uint16_t*)y + (size_t)t * d + n) = pk;
  } else {
    float* yp = (float*)y + (size_t)t * d + n;
    *(float4*)yp = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *(float4*)(yp + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_quantize_rows(const void* in, bool bf16, int64_t n_rows, int n_cols, uint8_t* codes, float* scales,
                                hipStream_t st) {
  const int gpr = n_cols / 128;
  const int64_t blocks = (n_rows + 3) / 4;
  if (bf16) quantize_rows_kernel<true><<<(unsigned)blocks, 256, 0, st>>>(in, n_rows, gpr, codes, scales);
  else quantize_rows_kernel<false><<<(unsigned)blocks, 256, 0, st>>>(in, n_rows, gpr, codes, scales);
  return hipGetLastError();
}

template <typename K>
static hipError_t launch_dyn(K kernel, dim3 grid, size_t lds, hipStream_t st, const ExpertArgs& a,
                             int threads = 256) {
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kernel<<<grid, threads, lds, st>>>(a);
  return hipGetLastError();
}

// Activations in LDS as bf16 for 16-row tiles; taller FP8 tiles stage them as
// bf16 by parts of K (gateup_x_part_blocks), so that two blocks fit a CU.
static bool gateup_x_bf16(int BM, int wmode) { return wmode != 2 || BM <= 16; }

// wmode: the moe_dtype of the weights (0 f32, 1 bf16, 2 FP8, 3 FP8 as W8A16,
// 4 4-bit groups).
size_t gateup_lds_bytes(int BM, int wmode, int d) {
  if (wmode == 0) return 1;  // static LDS only
  if (wmode == 4) return (size_t)(BM + 1) * (d * 2 + kLdsRowPad) + (size_t)(d / 64) * BM * 4;
  const int xrow = gateup_x_bf16(BM, wmode) ? d * 2 : gateup_x_part_blocks(d / 128) * 256;
  size_t b = (size_t)(BM + 1) * (xrow + kLdsRowPad);  // plus a spare row
  if (wmode >= 2) b += 2 * (size_t)BM * (d / 128) * 4;  // scale products
  return b + kGateUpWaves * BM * 4;
}

size_t down_lds_bytes(int BM, int wmode, int Fg) {
  if (wmode == 0) return 1;  // static LDS only
  if (wmode == 4) return (size_t)(BM + 1) * (Fg * 2 + kLdsRowPad) + (size_t)(Fg / 64) * BM * 4 + BM * 4 + BM * 4;
  size_t b = (size_t)(BM + 1) * (Fg * 2 + kLdsRowPad);  // h as bf16, plus a spare row
  if (wmode >= 2) b += (size_t)BM * (Fg / 128) * 4 + 2 * (Fg / 128) * 4;
  return b + BM * 4 + BM * 4;
}

// Tiles, slices and schedule sizes of one forward call.
int down_rows_per_wave(int BM, int wmode, int Fmax, int d) {
  // RT 16-row weight tiles per wave (RT > 1 needs a row's whole K in one stage):
  // 2 for short tiles, 4 for tall ones, whose h rows are then staged once per
  // 256 output features
  if (wmode == 0) return 1;
  if (wmode == 4) return Fmax <= 5 * 128 ? 2 : 1;
  const bool one_stage = Fmax * (wmode >= 2 ? 1 : 2) <= 5 * 128;
  return !one_stage ? 1 : (BM == 16 ? (d % 128 == 0 ? 2 : 1) : (d % 256 == 0 ? 4 : 1));
}

void plan_sizes(int wmode, int BM, int max_tiles, int Fmax, int d, int& nsl_gu, int& nsl_dn, int& n_gu, int& n_dn) {
  const int RT = down_rows_per_wave(BM, wmode, Fmax, d);
  nsl_gu = wmode == 0 ? (Fmax + 63) / 64 : Fmax / 128;
  nsl_dn = (d + 64 * RT - 1) / (64 * RT);
  n_gu = (max_tiles * nsl_gu + 7) / 8 * 8;
  n_dn = (max_tiles * nsl_dn + 7) / 8 * 8;
}

hipError_t launch_gateup(const ExpertArgs& a0, int wmode, const Plan& plan, hipStream_t st) {
  ExpertArgs a = a0;
  a.sched = plan.sched[0];
  a.per_tile = !plan.xcd;
  a.nsl = plan.n_slices[0];
  const dim3 grid(plan.n_sched[0]);
  const int BM = plan.BM;
  if (wmode == 0) return launch_dyn(gateup_f32_kernel<16>, grid, gateup_lds_bytes(16, 0, a.d), st, a);
  const size_t lds = gateup_lds_bytes(BM, wmode, a.d);
  const int nt = kGateUpWaves * 64;
  if (wmode == 2 && BM == 16) return launch_dyn(gateup_mfma_kernel<16, 2, true>, grid, lds, st, a, nt);
  if (wmode == 2 && BM == 32) return launch_dyn(gateup_mfma_kernel<32, 2, false>, grid, lds, st, a, nt);
  if (wmode == 1 && BM == 16) return launch_dyn(gateup_mfma_kernel<16, 1, true>, grid, lds, st, a, nt);
  if (wmode == 3 && BM == 16) return launch_dyn(gateup_mfma_kernel<16, 2, true, true>, grid, lds, st, a, nt);
  if (wmode == 4 && BM == 16) return launch_dyn(gateup_u4_kernel<false>, grid, lds, st, a, nt);
  return hipErrorInvalidValue;
}

bool experts_fusable(int wmode, const Plan& plan, int Fmax, int d) {
  return wmode >= 2 && wmode <= 4 && plan.BM == 16 && !plan.xcd && plan.sync &&
         down_rows_per_wave(16, wmode, Fmax, d) == 2 && d % (kGateUpWaves * 32) == 0;
}

hipError_t launch_experts_fused(const ExpertArgs& a0, int wmode, const Plan& plan, int32_t* status, int32_t* sticky,
                                bool test_timeout, hipStream_t st) {
  ExpertArgs gu = a0, dn = a0;
  gu.sched = dn.sched = plan.sched[0];
  gu.per_tile = dn.per_tile = 1;
  gu.nsl = plan.n_slices[0];
  dn.nsl = a0.d / (kGateUpWaves * 32);  // 8 waves x 2 tiles x 16 features per down block
  const int Fmax = a0.F > a0.Fs ? a0.F : a0.Fs;
  const int n_gu = plan.max_tiles * gu.nsl, n_dn = plan.max_tiles * dn.nsl;
  size_t lds = gateup_lds_bytes(16, wmode, a0.d);
  const size_t ldn = down_lds_bytes(16, wmode, Fmax);
  if (ldn > lds) lds = ldn;
  auto kernel = wmode == 4 ? experts_fused_kernel<4> : wmode == 3 ? experts_fused_kernel<3> : experts_fused_kernel<2>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kernel<<<n_gu + n_dn, kGateUpWaves * 64, lds, st>>>(gu, dn, n_gu, plan.sync, plan.sync + plan.max_tiles, status,
                                                      sticky, test_timeout ? 1 : 0, test_timeout ? 16 : kSpinLimit);
  return hipGetLastError();
}

hipError_t launch_down(const ExpertArgs& a0, int wmode, const Plan& plan, hipStream_t st) {
  ExpertArgs a = a0;
  a.sched = plan.xcd ? plan.sched[1] : plan.sched[0];
  a.per_tile = !plan.xcd;
  a.nsl = plan.n_slices[1];
  const dim3 grid(plan.n_sched[1]);
  const int BM = plan.BM;
  const int Fmax = a.F > a.Fs ? a.F : a.Fs;
  if (wmode == 0) return launch_dyn(down_f32_kernel<16>, grid, down_lds_bytes(16, 0, Fmax), st, a);
  const size_t lds = down_lds_bytes(BM, wmode, Fmax);
  const int RT = down_rows_per_wave(BM, wmode, Fmax, a.d);
  if (wmode == 2 && RT == 2 && BM == 16) return launch_dyn(down_mfma_kernel<16, 2, 2>, grid, lds, st, a);
  if (wmode == 3 && RT == 2 && BM == 16) return launch_dyn(down_mfma_kernel<16, 2, 2, true>, grid, lds, st, a);
  if (wmode == 4 && RT == 2 && BM == 16) return launch_dyn(down_u4_kernel<2>, grid, lds, st, a);
  if (wmode == 4 && RT == 1 && BM == 16) return launch_dyn(down_u4_kernel<1>, grid, lds, st, a);
  if (wmode == 2 && RT == 4 && BM == 32) return launch_dyn(down_mfma_kernel<32, 2, 4>, grid, lds, st, a);
  if (RT != 1) return hipErrorInvalidValue;
  if (wmode == 2 && BM == 16) return launch_dyn(down_mfma_kernel<16, 2, 1>, grid, lds, st, a);
  if (wmode == 2 && BM == 32) return launch_dyn(down_mfma_kernel<32, 2, 1>, grid, lds, st, a);
  if (wmode == 1 && BM == 16) return launch_dyn(down_mfma_kernel<16, 1, 1>, grid, lds, st, a);
  if (wmode == 3 && BM == 16) return launch_dyn(down_mfma_kernel<16, 2, 1, true>, grid, lds, st, a);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Weight packing into MOE_LAYOUT_TILED: one thread per 16-byte slot; writes are
// consecutive, reads gather 16 rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ in, uint8_t* __restrict__ out,
                                                           int64_t n_slots, int rows, int row_bytes) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_slots) return;
  const int nkb = row_bytes / 128;
  const int64_t mat_slots = (int64_t)rows * row_bytes / 16;
  const int64_t m = i / mat_slots;
  const int64_t r = i - m * mat_slots;  // slot within the matrix
  const int64_t tile = r / 128;         // 2 KB = 128 slots per tile
  const int s = (int)(r % 128), h = s / 64, l = s % 64;
  const int rt = (int)(tile / nkb), kb = (int)(tile % nkb);
  const int row = rt * 16 + (l & 15), byte = kb * 128 + (l >> 4) * 16 + h * 64;
  const uint8_t* src = in + m * rows * (int64_t)row_bytes + (int64_t)row * row_bytes + byte;
  *(v4i*)(out + i * 16) = *(const v4i*)src;
}

hipError_t launch_pack_weights(int64_t n_mats, int rows, int row_bytes, const void* in, void* out, hipStream_t st) {
  const int64_t n_slots = n_mats * rows * (int64_t)row_bytes / 16;
  const int64_t blocks = (n_slots + 255) / 256;
  pack_weights_kernel<<<(unsigned)blocks, 256, 0, st>>>((const uint8_t*)in, (uint8_t*)out, n_slots, rows, row_bytes);
  return hipGetLastError();
}

// 4-bit weights into MOE_LAYOUT_TILED.  Codes: one thread per 4-byte output
// word -- word m of slot l in tile (rt, kb) holds row 16*rt + l%16, columns
// 128*kb + 32*m + 8*(l/16) + [0, 8), nibble j < 4 the even column 2j of them
// and nibble 4 + j the odd column 2j + 1.  Group parameters: one thread per
// (tile, block, row) entry of 8 bytes -- bf16 (scale, bias) of group 2*kb, then
// of group 2*kb + 1.
__global__ __launch_bounds__(256) void pack_u4_codes_kernel(const uint8_t* __restrict__ in,
                                                            uint32_t* __restrict__ out, int64_t n_words, int rows,
                                                            int cols) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_words) return;
  const int nkb = cols / 128;
  const int64_t mat_words = (int64_t)rows * cols / 8;
  const int64_t m = i / mat_words, r = i - m * mat_words;
  const int64_t blk = r / 256;  // 1 KB = 256 words per tile block
  const int w = (int)(r % 256), l = w / 4, word = w % 4;
  const int rt = (int)(blk / nkb), kb = (int)(blk % nkb);
  const int row = rt * 16 + (l & 15), col = kb * 128 + 32 * word + 8 * (l >> 4);
  const uint8_t* src = in + (m * rows + row) * (int64_t)(cols / 2) + col / 2;
  uint32_t o = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // source byte j: column col + 2j (low nibble), col + 2j + 1 (high)
    const uint32_t byte = src[j];
    o |= (byte & 0xFu) << (4 * j);
    o |= (byte >> 4) << (16 + 4 * j);
  }
  out[i] = o;
}

__global__ __launch_bounds__(256) void pack_u4_params_kernel(const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ biases,
                                                             uint2* __restrict__ out, int64_t n, int rows, int cols) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int nkb = cols / 128, ng = cols / 64;
  const int64_t per_mat = (int64_t)rows * nkb;
  const int64_t m = i / per_mat, e = i - m * per_mat;
  const int r = (int)(e % 16);
  const int64_t tb = e / 16;
  const int rt = (int)(tb / nkb), kb = (int)(tb % nkb);
  const int64_t src = (m * rows + rt * 16 + r) * (int64_t)ng + 2 * kb;
  uint2 v;
  v.x = (uint32_t)scales[src] | ((uint32_t)biases[src] << 16);
  v.y = (uint32_t)scales[src + 1] | ((uint32_t)biases[src + 1] << 16);
  out[i] = v;
}

hipError_t launch_pack_u4(int64_t n_mats, int rows, int cols, const void* codes, const void* scales,
                          const void* biases, void* codes_out, void* params_out, hipStream_t st) {
  const int64_t n_words = n_mats * rows * (int64_t)cols / 8;
  const int64_t n_par = n_mats * rows * (int64_t)(cols / 128);
  pack_u4_codes_kernel<<<(unsigned)((n_words + 255) / 256), 256, 0, st>>>((const uint8_t*)codes,
                                                                          (uint32_t*)codes_out, n_words, rows, cols);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  pack_u4_params_kernel<<<(unsigned)((n_par + 255) / 256), 256, 0, st>>>(
      (const uint16_t*)scales, (const uint16_t*)biases, (uint2*)params_out, n_par, rows, cols);
  return hipGetLastError();
}

hipError_t launch_combine(const float* part, const int32_t* idx, int T, int k, int d, int E, int P, bool has_shared,
                          void* y, bool bf16_out, hipStream_t st) {
  const int64_t n = (int64_t)T * (d / 8);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  constexpr int64_t kLastLevelCache = 256ll << 20;
  const bool nt = (int64_t)(P + T) * d * 4 > kLastLevelCache;
  const int hs = has_shared ? 1 : 0;
  if (bf16_out && nt) combine_kernel<true, true><<<blocks, 256, 0, st>>>(part, idx, T, k, d, E, P, hs, y);
  else if (bf16_out) combine_kernel<true, false><<<blocks, 256, 0, st>>>(part, idx, T, k, d, E, P, hs, y);
  else combine_kernel<false, false><<<blocks, 256, 0, st>>>(part, idx, T, k, d, E, P, hs, y);
  return hipGetLastError();
}

}  // namespace moe
