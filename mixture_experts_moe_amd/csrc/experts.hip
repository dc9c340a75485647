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
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Activation quantisation: per row and 128-element group, s = amax/448 (1 for
// an all-zero group), code = E4M3(v/s) round-to-nearest-even, saturating.  One
// wave per group, two elements per lane.
// ---------------------------------------------------------------------------
template <bool BF16IN>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const void* __restrict__ in, int64_t n_groups, int gpr,
                                                             uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= n_groups) return;
  const int64_t row = g / gpr, col = (g % gpr) * 128 + 2 * lane;
  const int64_t o = row * (int64_t)gpr * 128 + col;
  float v0, v1;
  if (BF16IN) {
    const uint32_t pr = *(const uint32_t*)((const uint16_t*)in + o);
    v0 = __uint_as_float(pr << 16);
    v1 = __uint_as_float(pr & 0xffff0000u);
  } else {
    const float2 pr = *(const float2*)((const float*)in + o);
    v0 = pr.x;
    v1 = pr.y;
  }
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  *(uint16_t*)(codes + o) = (uint16_t)pack2_e4m3(v0 / s, v1 / s);
  if (lane == 0) scales[g] = s;
}

// ---------------------------------------------------------------------------
// Tile plan: tiles per group = ceil(rows / BM); groups in order; one block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void plan_tiles_kernel(const int32_t* __restrict__ counts, int E, int T,
                                                           int has_shared, int BM, int2* __restrict__ tiles,
                                                           int32_t* __restrict__ tile_count) {
  __shared__ int32_t tmp[17];
  const int G = E + (has_shared ? 1 : 0);
  // each thread owns groups 2*tid and 2*tid + 1 (G <= 2048)
  int nt[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = 2 * threadIdx.x + i;
    int rows = 0;
    if (g < E) rows = counts[g];
    else if (g < G) rows = T;
    nt[i] = (rows + BM - 1) / BM;
  }
  int total;
  const int start = block1024_excl_scan(nt[0] + nt[1], tmp, &total);
  int s = start;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = 2 * threadIdx.x + i;
    for (int j = 0; j < nt[i]; ++j) tiles[s + j] = make_int2(g, j * BM);
    s += nt[i];
  }
  if (threadIdx.x == 0) *tile_count = total;
}

// Rows of one tile: for each of its BM rows, the activation (token) row, the
// output row of h (sorted pair index, or P + t for the shared expert), the
// partial-output row (pair index p, or P + t) and the routing weight.
struct TileRows {
  int g, m0, rows;
  bool shared;
};

__device__ __forceinline__ TileRows tile_rows(const ExpertArgs& a, int tile, int BM) {
  const int2 td = a.tiles[tile];
  TileRows r;
  r.g = td.x;
  r.m0 = td.y;
  r.shared = td.x == a.E;
  const int n = r.shared ? a.T : a.offsets[td.x + 1] - a.offsets[td.x];
  r.rows = min(BM, n - td.y);
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
// Block = 256 threads = 4 waves; blockIdx.x = 128-feature slice nb of h,
// blockIdx.y = tile.  Wave w owns h features nb*128 + w*32 + [0, 32): two
// 16-row tiles of W_gate and the same two of W_up, so g and u of a feature meet
// in one lane.
// ---------------------------------------------------------------------------
template <int BM, int WT>
__global__ __launch_bounds__(256) void gateup_mfma_kernel(ExpertArgs a) {
  constexpr int NC = BM / 16;
  constexpr int EB = WT == 2 ? 1 : 2;  // bytes per element
  const int tile = blockIdx.y;
  if (tile >= *a.tile_count) return;
  const TileRows tr = tile_rows(a, tile, BM);
  const int Fg = tr.shared ? a.Fs : a.F;
  const int nb = blockIdx.x;
  if (nb * 128 >= Fg) return;

  const int RB = a.d * EB;        // bytes per activation / weight row
  const int nbb = RB / 128;       // 128-byte K blocks
  const int xstride = RB + 16;    // padded LDS row
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* xs = smem;
  float* sxs = (float*)(smem + BM * xstride);       // [BM][d/128] (FP8 only)
  float* red = sxs + (WT == 2 ? BM * (a.d / 128) : 0);  // [4][BM]
  int* tok = (int*)(red + 4 * BM);                  // [BM] token of each row

  const int tid = threadIdx.x;
  if (tid < BM) {
    int t = -1;
    if (tid < tr.rows) t = tr.shared ? tr.m0 + tid : a.perm[a.offsets[tr.g] + tr.m0 + tid] / a.k;
    tok[tid] = t;
  }
  __syncthreads();
  {
    const int cpr = RB / 16;
    const uint8_t* xa = (const uint8_t*)a.xa;
    for (int i = tid; i < BM * cpr; i += 256) {
      const int r = i / cpr, c = i - r * cpr, t = tok[r];
      v4i v = {0, 0, 0, 0};
      if (t >= 0) v = *(const v4i*)(xa + (size_t)t * RB + c * 16);
      *(v4i*)(xs + r * xstride + c * 16) = v;
    }
    if (WT == 2) {
      const int nkb = a.d / 128;
      for (int i = tid; i < BM * nkb; i += 256) {
        const int r = i / nkb, c = i - r * nkb, t = tok[r];
        sxs[i] = t >= 0 ? a.sxa[(size_t)t * nkb + c] : 0.f;
      }
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lk = (lane >> 4) * 16;
  const size_t wsz = (size_t)a.F * RB;  // bytes of one routed expert matrix
  const uint8_t* wg = tr.shared ? (const uint8_t*)a.shg : (const uint8_t*)a.wg + (size_t)tr.g * wsz;
  const uint8_t* wu = tr.shared ? (const uint8_t*)a.shu : (const uint8_t*)a.wu + (size_t)tr.g * wsz;
  const int frow = nb * 128 + wave * 32;
  const uint8_t* pa[4] = {wg + (size_t)(frow + lr) * RB + lk, wg + (size_t)(frow + 16 + lr) * RB + lk,
                          wu + (size_t)(frow + lr) * RB + lk, wu + (size_t)(frow + 16 + lr) * RB + lk};
  const float* sgp = nullptr;
  const float* sup = nullptr;
  if (WT == 2) {
    const int nkb = a.d / 128;
    const size_t ssz = (size_t)(a.F / 128) * nkb;
    sgp = (tr.shared ? a.ssg : a.sg + (size_t)tr.g * ssz) + (size_t)nb * nkb;
    sup = (tr.shared ? a.ssu : a.su + (size_t)tr.g * ssz) + (size_t)nb * nkb;
  }

  v4f acc[4][NC];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i wlo[2][4], whi[2][4];
  auto load = [&](int s, int bb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      wlo[s][r] = __builtin_nontemporal_load((const v4i*)(pa[r] + bb * 128));
      whi[s][r] = __builtin_nontemporal_load((const v4i*)(pa[r] + bb * 128 + 64));
    }
  };
  auto compute = [&](int s, int bb) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint8_t* bp = xs + (c * 16 + lr) * xstride + bb * 128 + lk;
      const v4i blo = *(const v4i*)bp;
      const v4i bhi = *(const v4i*)(bp + 64);
      if constexpr (WT == 2) {
        const float sx = sxs[(c * 16 + lr) * nbb + bb];
        const float cg = sx * sgp[bb], cu = sx * sup[bb];
        v4i b[4];
        e4m3x16_to_bf16(blo, b[0], b[1]);
        e4m3x16_to_bf16(bhi, b[2], b[3]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const v4f p = kblock_e4m3_exact(wlo[s][r], whi[s][r], b);
          const float cs = r < 2 ? cg : cu;
          acc[r][c] += p * cs;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[r][c] = mfma_bf16(wlo[s][r], blo, acc[r][c]);
          acc[r][c] = mfma_bf16(whi[s][r], bhi, acc[r][c]);
        }
      }
    }
  };
  load(0, 0);
  if (nbb > 1) load(1, 1);
  for (int bb = 0; bb < nbb; bb += 2) {
    compute(0, bb);
    if (bb + 2 < nbb) load(0, bb + 2);
    if (bb + 1 < nbb) {
      compute(1, bb + 1);
      if (bb + 3 < nbb) load(1, bb + 3);
    }
  }

  // Epilogue: h = silu(g) * u for features frow + r*16 + 4*(lane/16) + i, row c*16 + lane%16.
  float h[2][NC][4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gv = acc[r][c][i], uv = acc[2 + r][c][i];
        h[r][c][i] = gv / (1.0f + expf(-gv)) * uv;
      }
  const int hrow0 = tr.shared ? a.P + tr.m0 : a.offsets[tr.g] + tr.m0;
  if constexpr (WT == 2) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(h[r][c][i]));
      m = fmaxf(m, __shfl_xor(m, 16, kWave));
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      if (lane < 16) red[wave * BM + c * 16 + lane] = m;
    }
    __syncthreads();
    uint8_t* hq = (uint8_t*)a.h;
    const int gpr = a.hstride / 128;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int rr = c * 16 + lr;
      const float amax = fmaxf(fmaxf(red[rr], red[BM + rr]), fmaxf(red[2 * BM + rr], red[3 * BM + rr]));
      const float s = amax > 0.f ? amax / 448.0f : 1.0f;
      if (rr < tr.rows) {
        const size_t row = (size_t)(hrow0 + rr);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint32_t pk = pack4_e4m3(h[r][c][0] / s, h[r][c][1] / s, h[r][c][2] / s, h[r][c][3] / s);
          *(uint32_t*)(hq + row * a.hstride + frow + r * 16 + 4 * (lane >> 4)) = pk;
        }
        if (wave == 0 && lane < 16) a.sh[row * gpr + nb] = s;
      }
    }
  } else {
    uint16_t* hb = (uint16_t*)a.h;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int rr = c * 16 + lr;
      if (rr < tr.rows) {
        const size_t row = (size_t)(hrow0 + rr);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16(h[r][c][0]) | ((uint32_t)f32_to_bf16(h[r][c][1]) << 16);
          pk.y = (uint32_t)f32_to_bf16(h[r][c][2]) | ((uint32_t)f32_to_bf16(h[r][c][3]) << 16);
          *(uint2*)(hb + row * a.hstride + frow + r * 16 + 4 * (lane >> 4)) = pk;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection on the matrix cores; epilogue multiplies by the pair's
// routing weight (1 for the shared expert) and writes the fp32 partial row of
// pair p (or P + t).  blockIdx.x = 256-feature slice of d, blockIdx.y = tile;
// wave w owns output features nb*256 + w*64 + [0, 64) as four 16-row tiles.
// ---------------------------------------------------------------------------
template <int BM, int WT>
__global__ __launch_bounds__(256) void down_mfma_kernel(ExpertArgs a) {
  constexpr int NC = BM / 16;
  constexpr int EB = WT == 2 ? 1 : 2;
  const int tile = blockIdx.y;
  if (tile >= *a.tile_count) return;
  const TileRows tr = tile_rows(a, tile, BM);
  const int nb = blockIdx.x;
  const int Fg = tr.shared ? a.Fs : a.F;
  const int RB = Fg * EB;          // bytes per h row / W_down row
  const int nbb = RB / 128;
  const int hstride_b = a.hstride * EB;
  const int lstride = RB + 16;
  extern __shared__ __align__(16) uint8_t smem[];
  uint8_t* hs = smem;
  float* shs = (float*)(smem + BM * lstride);                // [BM][Fg/128] (FP8)
  float* wrow = shs + (WT == 2 ? BM * (Fg / 128) : 0);       // [BM] routing weight
  int* orow = (int*)(wrow + BM);                             // [BM] partial-output row

  const int tid = threadIdx.x;
  const int hrow0 = tr.shared ? a.P + tr.m0 : a.offsets[tr.g] + tr.m0;
  if (tid < BM) {
    int o = -1;
    float w = 0.f;
    if (tid < tr.rows) {
      if (tr.shared) {
        o = a.P + tr.m0 + tid;
        w = 1.f;
      } else {
        o = a.perm[hrow0 + tid];
        w = a.topk_w[o];
      }
    }
    orow[tid] = o;
    wrow[tid] = w;
  }
  {
    const int cpr = RB / 16;
    const uint8_t* hsrc = (const uint8_t*)a.h;
    for (int i = tid; i < BM * cpr; i += 256) {
      const int r = i / cpr, c = i - r * cpr;
      v4i v = {0, 0, 0, 0};
      if (r < tr.rows) v = *(const v4i*)(hsrc + (size_t)(hrow0 + r) * hstride_b + c * 16);
      *(v4i*)(hs + r * lstride + c * 16) = v;
    }
    if (WT == 2) {
      const int nkb = Fg / 128, gpr = a.hstride / 128;
      for (int i = tid; i < BM * nkb; i += 256) {
        const int r = i / nkb, c = i - r * nkb;
        shs[i] = r < tr.rows ? a.sh[(size_t)(hrow0 + r) * gpr + c] : 0.f;
      }
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lk = (lane >> 4) * 16;
  if (nb * 256 + wave * 64 >= a.d) return;  // d is a multiple of 64: whole waves drop out
  const uint8_t* wd = tr.shared ? (const uint8_t*)a.shd : (const uint8_t*)a.wd + (size_t)tr.g * a.d * RB;
  const int n0 = nb * 256 + wave * 64;
  const uint8_t* pa[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pa[r] = wd + (size_t)(n0 + r * 16 + lr) * RB + lk;
  const float* sdp[4] = {nullptr, nullptr, nullptr, nullptr};
  if (WT == 2) {
    const int nkb = Fg / 128;
    const float* base = tr.shared ? a.ssd : a.sd + (size_t)tr.g * (a.d / 128) * nkb;
#pragma unroll
    for (int r = 0; r < 4; ++r) sdp[r] = base + (size_t)((n0 + r * 16) / 128) * nkb;
  }

  v4f acc[4][NC];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[r][c] = v4f{0.f, 0.f, 0.f, 0.f};
  v4i wlo[2][4], whi[2][4];
  auto load = [&](int s, int bb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      wlo[s][r] = __builtin_nontemporal_load((const v4i*)(pa[r] + bb * 128));
      whi[s][r] = __builtin_nontemporal_load((const v4i*)(pa[r] + bb * 128 + 64));
    }
  };
  auto compute = [&](int s, int bb) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint8_t* bp = hs + (c * 16 + lr) * lstride + bb * 128 + lk;
      const v4i blo = *(const v4i*)bp;
      const v4i bhi = *(const v4i*)(bp + 64);
      if constexpr (WT == 2) {
        const float sx = shs[(c * 16 + lr) * nbb + bb];
        v4i b[4];
        e4m3x16_to_bf16(blo, b[0], b[1]);
        e4m3x16_to_bf16(bhi, b[2], b[3]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const v4f p = kblock_e4m3_exact(wlo[s][r], whi[s][r], b);
          acc[r][c] += p * (sx * sdp[r][bb]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          acc[r][c] = mfma_bf16(wlo[s][r], blo, acc[r][c]);
          acc[r][c] = mfma_bf16(whi[s][r], bhi, acc[r][c]);
        }
      }
    }
  };
  load(0, 0);
  if (nbb > 1) load(1, 1);
  for (int bb = 0; bb < nbb; bb += 2) {
    compute(0, bb);
    if (bb + 2 < nbb) load(0, bb + 2);
    if (bb + 1 < nbb) {
      compute(1, bb + 1);
      if (bb + 3 < nbb) load(1, bb + 3);
    }
  }

#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int rr = c * 16 + lr;
    if (rr < tr.rows) {
      const float w = wrow[rr];
      float* dst = a.part + (size_t)orow[rr] * a.d + n0 + 4 * (lane >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const v4f v = acc[r][c] * w;
        *(float4*)(dst + r * 16) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 expert projections (fp32 activations and weights): plain fp32
// multiply-add, one output feature per thread.  blockIdx.x = 64-feature slice.
// ---------------------------------------------------------------------------
template <int BM>
__global__ __launch_bounds__(256) void gateup_f32_kernel(ExpertArgs a) {
  const int tile = blockIdx.y;
  if (tile >= *a.tile_count) return;
  const TileRows tr = tile_rows(a, tile, BM);
  const int Fg = tr.shared ? a.Fs : a.F;
  const int f = blockIdx.x * 64 + (threadIdx.x & 63);
  if (blockIdx.x * 64 >= Fg) return;
  extern __shared__ __align__(16) uint8_t smem[];
  float* xs = (float*)smem;  // [BM][d]
  const int tid = threadIdx.x;
  const float* x = (const float*)a.xa;
  for (int i = tid; i < BM * a.d; i += 256) {
    const int r = i / a.d, c = i - r * a.d;
    float v = 0.f;
    if (r < tr.rows) {
      const int t = tr.shared ? tr.m0 + r : a.perm[a.offsets[tr.g] + tr.m0 + r] / a.k;
      v = x[(size_t)t * a.d + c];
    }
    xs[i] = v;
  }
  __syncthreads();
  if (f >= Fg) return;
  const size_t wsz = (size_t)a.F * a.d;
  const float* wg = (tr.shared ? (const float*)a.shg : (const float*)a.wg + tr.g * wsz) + (size_t)f * a.d;
  const float* wu = (tr.shared ? (const float*)a.shu : (const float*)a.wu + tr.g * wsz) + (size_t)f * a.d;
  const int hrow0 = tr.shared ? a.P + tr.m0 : a.offsets[tr.g] + tr.m0;
  for (int r = tid >> 6; r < tr.rows; r += 4) {
    float g = 0.f, u = 0.f;
    for (int c = 0; c < a.d; ++c) {
      g = fmaf(wg[c], xs[r * a.d + c], g);
      u = fmaf(wu[c], xs[r * a.d + c], u);
    }
    ((float*)a.h)[(size_t)(hrow0 + r) * a.hstride + f] = g / (1.0f + expf(-g)) * u;
  }
}

template <int BM>
__global__ __launch_bounds__(256) void down_f32_kernel(ExpertArgs a) {
  const int tile = blockIdx.y;
  if (tile >= *a.tile_count) return;
  const TileRows tr = tile_rows(a, tile, BM);
  const int Fg = tr.shared ? a.Fs : a.F;
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  extern __shared__ __align__(16) uint8_t smem[];
  float* hs = (float*)smem;  // [BM][Fg]
  const int tid = threadIdx.x;
  const int hrow0 = tr.shared ? a.P + tr.m0 : a.offsets[tr.g] + tr.m0;
  for (int i = tid; i < BM * Fg; i += 256) {
    const int r = i / Fg, c = i - r * Fg;
    hs[i] = r < tr.rows ? ((const float*)a.h)[(size_t)(hrow0 + r) * a.hstride + c] : 0.f;
  }
  __syncthreads();
  if (n >= a.d) return;
  const float* wd = (tr.shared ? (const float*)a.shd : (const float*)a.wd + tr.g * (size_t)a.d * Fg) + (size_t)n * Fg;
  for (int r = tid >> 6; r < tr.rows; r += 4) {
    float acc = 0.f;
    for (int c = 0; c < Fg; ++c) acc = fmaf(wd[c], hs[r * Fg + c], acc);
    int o;
    float w;
    if (tr.shared) {
      o = a.P + tr.m0 + r;
      w = 1.f;
    } else {
      o = a.perm[hrow0 + r];
      w = a.topk_w[o];
    }
    a.part[(size_t)o * a.d + n] = acc * w;
  }
}

// ---------------------------------------------------------------------------
// Combine, fixed order per token: acc = shared; acc += (w_j * y_j) for
// j = 0..k-1 (the products were formed in the down epilogue); y = round(acc).
// Invalid slots (id -1) are skipped.  Four features per thread.
// ---------------------------------------------------------------------------
template <bool BF16OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part,
                                                      const int32_t* __restrict__ idx, int T, int k, int d, int E,
                                                      int P, int has_shared, void* __restrict__ y) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q = d / 4;
  if (gid >= (int64_t)T * q) return;
  const int t = (int)(gid / q), n = (int)(gid - (int64_t)t * q) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (has_shared) acc = *(const float4*)(part + (size_t)(P + t) * d + n);
  for (int j = 0; j < k; ++j) {
    const int e = idx[(size_t)t * k + j];
    if (e < 0 || e >= E) continue;
    const float4 v = *(const float4*)(part + ((size_t)t * k + j) * d + n);
    acc.x = acc.x + v.x;
    acc.y = acc.y + v.y;
    acc.z = acc.z + v.z;
    acc.w = acc.w + v.w;
  }
  if (BF16OUT) {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    pk.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    *(uint2*)((uint16_t*)y + (size_t)t * d + n) = pk;
  } else {
    *(float4*)((float*)y + (size_t)t * d + n) = acc;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_quantize_rows(const void* in, bool bf16, int64_t n_rows, int n_cols, uint8_t* codes, float* scales,
                                hipStream_t st) {
  const int gpr = n_cols / 128;
  const int64_t ng = n_rows * gpr;
  const int64_t blocks = (ng + 3) / 4;
  if (bf16) quantize_rows_kernel<true><<<(unsigned)blocks, 256, 0, st>>>(in, ng, gpr, codes, scales);
  else quantize_rows_kernel<false><<<(unsigned)blocks, 256, 0, st>>>(in, ng, gpr, codes, scales);
  return hipGetLastError();
}

hipError_t launch_plan_tiles(const int32_t* counts, int E, int T, bool has_shared, int BM, int2* tiles,
                             int32_t* tile_count, hipStream_t st) {
  plan_tiles_kernel<<<1, 1024, 0, st>>>(counts, E, T, has_shared ? 1 : 0, BM, tiles, tile_count);
  return hipGetLastError();
}

template <typename K>
static hipError_t launch_dyn(K kernel, dim3 grid, size_t lds, hipStream_t st, const ExpertArgs& a) {
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kernel<<<grid, 256, lds, st>>>(a);
  return hipGetLastError();
}

size_t gateup_lds_bytes(int BM, int wmode, int d) {
  if (wmode == 0) return (size_t)BM * d * 4;
  const int EB = wmode == 2 ? 1 : 2;
  size_t b = (size_t)BM * (d * EB + 16);
  if (wmode == 2) b += (size_t)BM * (d / 128) * 4;
  return b + 4 * BM * 4 + BM * 4;
}

size_t down_lds_bytes(int BM, int wmode, int Fg) {
  if (wmode == 0) return (size_t)BM * Fg * 4;
  const int EB = wmode == 2 ? 1 : 2;
  size_t b = (size_t)BM * (Fg * EB + 16);
  if (wmode == 2) b += (size_t)BM * (Fg / 128) * 4;
  return b + BM * 4 + BM * 4;
}

hipError_t launch_gateup(const ExpertArgs& a, int wmode, int BM, int max_tiles, hipStream_t st) {
  const int Fmax = a.F > a.Fs ? a.F : a.Fs;
  if (wmode == 0)
    return launch_dyn(gateup_f32_kernel<16>, dim3((Fmax + 63) / 64, max_tiles), gateup_lds_bytes(16, 0, a.d), st, a);
  const dim3 grid(Fmax / 128, max_tiles);
  const size_t lds = gateup_lds_bytes(BM, wmode, a.d);
  if (wmode == 2 && BM == 16) return launch_dyn(gateup_mfma_kernel<16, 2>, grid, lds, st, a);
  if (wmode == 2 && BM == 32) return launch_dyn(gateup_mfma_kernel<32, 2>, grid, lds, st, a);
  if (wmode == 2 && BM == 64) return launch_dyn(gateup_mfma_kernel<64, 2>, grid, lds, st, a);
  if (wmode == 1 && BM == 16) return launch_dyn(gateup_mfma_kernel<16, 1>, grid, lds, st, a);
  return hipErrorInvalidValue;
}

hipError_t launch_down(const ExpertArgs& a, int wmode, int BM, int max_tiles, hipStream_t st) {
  const int Fmax = a.F > a.Fs ? a.F : a.Fs;
  if (wmode == 0)
    return launch_dyn(down_f32_kernel<16>, dim3((a.d + 63) / 64, max_tiles), down_lds_bytes(16, 0, Fmax), st, a);
  const dim3 grid((a.d + 255) / 256, max_tiles);
  const size_t lds = down_lds_bytes(BM, wmode, Fmax);
  if (wmode == 2 && BM == 16) return launch_dyn(down_mfma_kernel<16, 2>, grid, lds, st, a);
  if (wmode == 2 && BM == 32) return launch_dyn(down_mfma_kernel<32, 2>, grid, lds, st, a);
  if (wmode == 2 && BM == 64) return launch_dyn(down_mfma_kernel<64, 2>, grid, lds, st, a);
  if (wmode == 1 && BM == 16) return launch_dyn(down_mfma_kernel<16, 1>, grid, lds, st, a);
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const float* part, const int32_t* idx, int T, int k, int d, int E, int P, bool has_shared,
                          void* y, bool bf16_out, hipStream_t st) {
  const int64_t n = (int64_t)T * (d / 4);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (bf16_out) combine_kernel<true><<<blocks, 256, 0, st>>>(part, idx, T, k, d, E, P, has_shared ? 1 : 0, y);
  else combine_kernel<false><<<blocks, 256, 0, st>>>(part, idx, T, k, d, E, P, has_shared ? 1 : 0, y);
  return hipGetLastError();
}

}  // namespace moe
