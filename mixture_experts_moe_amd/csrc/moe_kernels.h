// Internal launch interface between the C ABI (moe_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 8;

// Per h row q (sorted pairs, then P + t for the shared expert): token, row of
// the partial output, routing weight (1 for the shared expert).
struct RowInfo {
  int32_t* tok;
  int32_t* prow;
  float* w;
};

// Schedule parameters of the dispatch plan (see moe_plan.h).
struct PlanArgs {
  const int32_t* counts;   // [E] pairs per expert
  const int32_t* offsets;  // [E] first sorted pair of each expert
  int E, T, P, has_shared, BM, xcd;
  int4* sched[2];          // gate/up, down (xcd: one record per block; else sched[0] is the tile list)
  int n_sched[2];          // blocks of each kernel
  int n_slices[2];
  int max_tiles;           // entries of the tile list
  int32_t* sync;           // [2][max_tiles] tile-list schedules: counters of the fused expert launch, zeroed here
};

// Where the routing call's last launch writes the dispatch plan, and the
// activations it quantises.
struct PlanCtx {
  PlanArgs pa;
  RowInfo ri;
  const uint16_t* x;  // bf16 activations [T][d] (quantised when xq != null)
  uint8_t* xq;
  float* sx;
  int n_rows;         // T when quantising, else 0
  int gpr;            // d / 128
  int k;
};

// Everything the expert kernels read or write (device pointers).
struct ExpertArgs {
  const int4* sched;          // per_tile: tile list (group, first row, first h row, rows), block b takes tile
                              // b / nsl and slice b % nsl; else one record per block with rows | slice << 16;
                              // group -1: no work
  int per_tile, nsl;          // set per launch
  const int32_t* offsets;     // [E+1]
  const int32_t* perm;        // [P]
  const float* topk_w;        // [P]
  int T, d, E, k, F, Fs, P;
  int hstride;                // elements per h row = max(F, Fs)
  int w_tiled;                // weights in MOE_LAYOUT_TILED
  const void* xa;             // gate/up input rows: E4M3 codes, bf16 or fp32 [T][d]
  const float* sxa;           // E4M3 activation scales [T][d/128]
  const void *wg, *wu, *wd;
  const float *sg, *su, *sd;
  const void *shg, *shu, *shd;
  const float *ssg, *ssu, *ssd;
  void* h;                    // [P+T][hstride]: E4M3 codes, bf16 or fp32
  float* sh;                  // [P+T][hstride/128] E4M3 scales of h
  float* part;                // [P+T][d] weighted expert outputs
  RowInfo ri;                 // [P+T] each
};

size_t dispatch_chunk_hist_ints(int T, int k, int E);
// Router partial sums kept between the router and top-k launches (bf16 activations).
size_t router_part_floats(int T, int k, int d, int E, bool x_bf16);

struct RouteLaunch {
  const void* x;
  bool x_bf16;
  const float* w_router;
  const uint8_t* planes;   // the router weights packed by launch_pack_router, or null
  const float* bias;       // selection bias or null
  const int32_t* forced;   // forced ids or null
  int T, d, E, k;
  float* logits;           // where the logits go (the caller's buffer or workspace)
  float* rpart;            // [d/kslice][T][E] router partial sums (bf16 activations)
  int32_t* idx;
  float* w;
  int32_t *chunk_hist, *local_rank, *counts, *offsets, *perm, *inv_perm, *status;
  PlanCtx plan;            // the dispatch plan the last launch writes
};
hipError_t launch_route(const RouteLaunch& L, hipStream_t st);
// The router weights [E][d] fp32 as three exact bf16 planes in matrix-core
// operand order (the layout is described at pack_router_planes_kernel).
size_t router_planes_bytes(int d, int E);
hipError_t launch_pack_router(const float* W, void* planes, int d, int E, hipStream_t st);

hipError_t launch_quantize_rows(const void* in, bool bf16, int64_t n_rows, int n_cols, uint8_t* codes, float* scales,
                                hipStream_t st);
// Block schedules of the two expert kernels ([0] gate/up, [1] down), written by
// the routing call: BM rows per tile.  xcd (experts with several tiles): one
// record per block, an expert's tiles kept on one XCD; otherwise the blocks
// take the tiles in order, slice fastest, from one shared tile list (sched[0]).
struct Plan {
  int BM;
  bool xcd;
  int4* sched[2];
  int n_sched[2];   // blocks of each kernel
  int n_slices[2];  // feature slices per tile
  int max_tiles;
  int32_t* sync;    // [2][max_tiles] per-tile counters (tile-list schedules only, else null)
};
int down_rows_per_wave(int BM, int wmode, int Fmax, int d);
void plan_sizes(int wmode, int BM, int max_tiles, int Fmax, int d, int& nsl_gu, int& nsl_dn, int& n_gu, int& n_dn);
hipError_t launch_gateup(const ExpertArgs& a, int wmode, const Plan& plan, hipStream_t st);
hipError_t launch_down(const ExpertArgs& a, int wmode, const Plan& plan, hipStream_t st);
// Gate/up and down as one launch (FP8 weights, 16-row tiles, tile-list plan).
bool experts_fusable(int wmode, const Plan& plan, int Fmax, int d);
// status: the routing status word; sticky: the caller's sticky forward status
// (or null); test_timeout: the waits target a count that never comes (error-path test).
hipError_t launch_experts_fused(const ExpertArgs& a, int wmode, const Plan& plan, int32_t* status, int32_t* sticky,
                                bool test_timeout, hipStream_t st);
hipError_t launch_pack_weights(int64_t n_mats, int rows, int row_bytes, const void* in, void* out,
                               hipStream_t st);
size_t route_compare_ws_bytes(int T);
hipError_t launch_route_compare(int T, int E, int k, const float* logits, const float* ref_logits, const float* bias,
                                const int32_t* idx, const int32_t* ref_idx, float* gap, double* sigma,
                                int32_t* n_differ, float* max_gap, void* ws, hipStream_t st);
hipError_t launch_pack_u4(int64_t n_mats, int rows, int cols, const void* codes, const void* scales,
                          const void* biases, void* codes_out, void* params_out, hipStream_t st);
hipError_t launch_combine(const float* part, const int32_t* idx, int T, int k, int d, int E, int P, bool has_shared,
                          void* y, bool bf16_out, hipStream_t st);
size_t gateup_lds_bytes(int BM, int wmode, int d);
size_t down_lds_bytes(int BM, int wmode, int Fg);

}  // namespace moe
