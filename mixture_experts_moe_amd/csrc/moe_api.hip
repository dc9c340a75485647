// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout, kernel launches on the caller's stream.  Holds no state,
// except the per-device address of the no-allocation forward's scratch buffer
// (resolved once per device, then only read).
#include <limits.h>

#include <atomic>
#include <mutex>

#include "moe.h"
#include "moe_kernels.h"

// Scratch of moe_forward_noalloc: the forward's h rows, their scales and the
// fp32 partials.  One copy per device the library runs on, held until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in for the symbol): it asks hipGetSymbolAddress for each
// device's copy once and passes that pointer to the kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

using moe::ExpertArgs;

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t logits, rpart, chunk_hist, local_rank, h, sh, part, total;
};

// Segments of the dispatch plan (moe_routing.plan), written by the routing call
// and read by the forward call.
struct PlanLayout {
  size_t sched_gu, sched_dn, rinfo, xq, sx, sync, total;
};

int h_elem_bytes(int w_dtype) { return w_dtype == MOE_FP8E4M3_B128 ? 1 : (w_dtype == MOE_F32 ? 4 : 2); }

int64_t max_tiles_for(const moe_shape& s, int BM) {
  const int64_t P = (int64_t)s.T * s.top_k;
  int64_t n = (P + BM - 1) / BM + (P < s.n_experts ? P : s.n_experts);
  if (s.d_ffn_shared > 0) n += (s.T + BM - 1) / BM;
  return n;
}

// Workspace segments (256-byte aligned).  Routing uses logits (when the caller
// passes none), the router partial sums, chunk_hist and local_rank; the forward
// pass uses the rest.  Nothing is carried from one call to the next: what the
// forward pass needs from routing travels in moe_routing (plan included).
// forward_only: the routing segments are empty (the no-allocation forward's
// scratch holds only the forward's segments).
Layout layout(const moe_shape& s, bool forward_only = false) {
  const size_t T = s.T, d = s.d_model, E = s.n_experts, P = T * s.top_k;
  const size_t Fmax = s.d_ffn > s.d_ffn_shared ? s.d_ffn : s.d_ffn_shared;
  const bool fp8 = s.w_dtype == MOE_FP8E4M3_B128;
  Layout L;
  size_t o = 0;
  auto seg = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  const size_t rt = forward_only ? 0 : 1;
  L.logits = seg(rt * T * E * 4);
  L.rpart = seg(rt * moe::router_part_floats(s.T, s.top_k, s.d_model, s.n_experts, s.act_dtype == MOE_BF16) * 4);
  L.chunk_hist = seg(rt * moe::dispatch_chunk_hist_ints(s.T, s.top_k, s.n_experts) * 4);
  L.local_rank = seg(rt * P * 4);
  L.h = seg((P + T) * Fmax * h_elem_bytes(s.w_dtype));
  L.sh = seg(fp8 ? (P + T) * (Fmax / 128) * 4 : 0);
  L.part = seg((P + T) * d * 4);
  L.total = o;
  return L;
}

PlanLayout plan_layout(const moe_shape& s) {
  const size_t T = s.T, d = s.d_model, P = T * s.top_k;
  const size_t Fmax = s.d_ffn > s.d_ffn_shared ? s.d_ffn : s.d_ffn_shared;
  const bool fp8 = s.w_dtype == MOE_FP8E4M3_B128;
  PlanLayout L;
  size_t o = 0;
  auto seg = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  // block schedules, sized for the largest case (16-row tiles, 64-feature slices)
  const size_t mt = (size_t)max_tiles_for(s, 16);
  L.sched_gu = seg((mt * ((Fmax + 63) / 64) + 7) / 8 * 8 * sizeof(int4));
  L.sched_dn = seg((mt * ((d + 63) / 64) + 7) / 8 * 8 * sizeof(int4));
  L.rinfo = seg((P + T) * 12);
  L.xq = seg(fp8 ? T * d : 0);
  L.sx = seg(fp8 ? T * (d / 128) * 4 : 0);
  L.sync = seg(2 * mt * 4);  // per tile: gate/up slices done, down blocks done (fused expert launch)
  L.total = o;
  return L;
}

int validate_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->T < 0 || s->d_model <= 0 || s->n_experts <= 0 || s->top_k <= 0 || s->d_ffn <= 0 || s->d_ffn_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->top_k > s->n_experts) return MOE_ERR_INVALID_ARG;
  if (s->top_k > moe::kMaxTopK || s->n_experts > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)s->T * s->top_k > INT_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const bool combo = (s->act_dtype == MOE_F32 && s->w_dtype == MOE_F32) ||
                     (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_BF16) ||
                     (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_FP8E4M3_B128) ||
                     (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_FP8E4M3_B128_A16) ||
                     (s->act_dtype == MOE_BF16 && s->w_dtype == MOE_U4_G64);
  if (!combo) return MOE_ERR_UNSUPPORTED;
  if (s->w_layout != MOE_LAYOUT_ROWMAJOR && s->w_layout != MOE_LAYOUT_TILED) return MOE_ERR_INVALID_ARG;
  if (s->w_layout == MOE_LAYOUT_TILED && s->w_dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (s->w_layout != MOE_LAYOUT_TILED && s->w_dtype == MOE_U4_G64) return MOE_ERR_UNSUPPORTED;
  if (s->d_model % 128 || s->d_ffn % 128 || s->d_ffn_shared % 128) return MOE_ERR_UNSUPPORTED;
  if (s->d_model > 8192 || s->d_ffn > 4096 || s->d_ffn_shared > 4096) return MOE_ERR_UNSUPPORTED;
  const int Fmax = s->d_ffn > s->d_ffn_shared ? s->d_ffn : s->d_ffn_shared;
  if (s->w_dtype == MOE_F32 && (s->d_model > 2560 || Fmax > 2560)) return MOE_ERR_UNSUPPORTED;  // documented limit
  if (moe::gateup_lds_bytes(16, s->w_dtype, s->d_model) > kMaxLds) return MOE_ERR_UNSUPPORTED;
  if (moe::down_lds_bytes(16, s->w_dtype, Fmax) > kMaxLds) return MOE_ERR_UNSUPPORTED;
  if (max_tiles_for(*s, 16) * (s->d_model / 64 + Fmax / 64 + 16) > INT_MAX / 2) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Rows per tile of the grouped expert GEMMs: more rows per expert -> taller
// tiles (weights re-streamed less often), within the LDS budget.
int pick_bm(const moe_shape& s) {
  if (s.w_dtype != MOE_FP8E4M3_B128) return 16;
  const int64_t per_expert = (int64_t)s.T * s.top_k / s.n_experts;
  int bm = per_expert <= 12 ? 16 : 32;
  const int Fmax = s.d_ffn > s.d_ffn_shared ? s.d_ffn : s.d_ffn_shared;
  while (bm > 16 && (moe::gateup_lds_bytes(bm, s.w_dtype, s.d_model) > kMaxLds ||
                     moe::down_lds_bytes(bm, s.w_dtype, Fmax) > kMaxLds))
    bm /= 2;
  return bm;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Each device's address of `scratch`, looked up on the first no-allocation
// call on that device (with that device current) and kept for the process.
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

// The kernels move 16 bytes per lane through every tensor.
bool misaligned(const void* p) { return ((uintptr_t)p & 15) != 0; }

int check_routing_out(const moe_routing* r) {
  if (!r || !r->topk_idx || !r->topk_w || !r->counts || !r->offsets || !r->perm || !r->inv_perm || !r->status ||
      !r->plan)
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// The plan of one call: tile height, schedule sizes and where its parts sit in
// the plan buffer (the same for the routing call that writes it and the forward
// call that reads it).
struct PlanView {
  moe::Plan plan;
  moe::RowInfo ri;
  uint8_t* xq;
  float* sx;
};

PlanView plan_view(const moe_shape& s, void* plan_buf) {
  const PlanLayout pl = plan_layout(s);
  char* base = (char*)plan_buf;
  const int P = s.T * s.top_k;
  const int Fmax = s.d_ffn > s.d_ffn_shared ? s.d_ffn : s.d_ffn_shared;
  PlanView v;
  v.plan.BM = pick_bm(s);
  v.plan.xcd = v.plan.BM > 16;  // several tiles per expert: keep an expert's tiles on one XCD
  moe::plan_sizes(s.w_dtype, v.plan.BM, (int)max_tiles_for(s, v.plan.BM), Fmax, s.d_model, v.plan.n_slices[0],
                  v.plan.n_slices[1], v.plan.n_sched[0], v.plan.n_sched[1]);
  v.plan.max_tiles = (int)max_tiles_for(s, v.plan.BM);
  if (!v.plan.xcd)  // blocks take the tiles in order from one tile list
    for (int i = 0; i < 2; ++i) v.plan.n_sched[i] = v.plan.max_tiles * v.plan.n_slices[i];
  v.plan.sched[0] = (int4*)(base + pl.sched_gu);
  v.plan.sched[1] = (int4*)(base + pl.sched_dn);
  v.plan.sync = v.plan.xcd ? nullptr : (int32_t*)(base + pl.sync);
  v.ri.tok = (int32_t*)(base + pl.rinfo);
  v.ri.prow = v.ri.tok + (P + s.T);
  v.ri.w = (float*)(v.ri.prow + (P + s.T));
  const bool fp8 = s.w_dtype == MOE_FP8E4M3_B128;
  v.xq = fp8 ? (uint8_t*)(base + pl.xq) : nullptr;
  v.sx = fp8 ? (float*)(base + pl.sx) : nullptr;
  return v;
}

int route_common(const moe_shape* shape, const moe_weights* w, const void* x, const int32_t* forced,
                 const moe_routing* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!w || !w->w_router || !x || check_routing_out(out) != MOE_OK) return MOE_ERR_INVALID_ARG;
  if (misaligned(x) || misaligned(w->w_router) || misaligned(w->w_router_planes)) return MOE_ERR_INVALID_ARG;
  if (shape->T == 0) return MOE_OK;
  if (!ws) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(*shape);
  if (ws_bytes < L.total || out->plan_bytes < plan_layout(*shape).total) return MOE_ERR_WORKSPACE;
  char* base = (char*)ws;
  moe::RouteLaunch R;
  R.x = x;
  R.x_bf16 = shape->act_dtype == MOE_BF16;
  R.w_router = w->w_router;
  R.planes = (const uint8_t*)w->w_router_planes;
  R.bias = w->sel_bias;
  R.forced = forced;
  R.T = shape->T;
  R.d = shape->d_model;
  R.E = shape->n_experts;
  R.k = shape->top_k;
  R.logits = out->logits ? out->logits : (float*)(base + L.logits);
  R.rpart = (float*)(base + L.rpart);
  R.idx = out->topk_idx;
  R.w = out->topk_w;
  R.chunk_hist = (int32_t*)(base + L.chunk_hist);
  R.local_rank = (int32_t*)(base + L.local_rank);
  R.counts = out->counts;
  R.offsets = out->offsets;
  R.perm = out->perm;
  R.inv_perm = out->inv_perm;
  R.status = out->status;
  const PlanView v = plan_view(*shape, out->plan);
  moe::PlanCtx& pc = R.plan;
  pc.pa.counts = out->counts;
  pc.pa.offsets = out->offsets;
  pc.pa.E = shape->n_experts;
  pc.pa.T = shape->T;
  pc.pa.P = shape->T * shape->top_k;
  pc.pa.has_shared = shape->d_ffn_shared > 0 ? 1 : 0;
  pc.pa.BM = v.plan.BM;
  pc.pa.xcd = v.plan.xcd ? 1 : 0;
  for (int i = 0; i < 2; ++i) {
    pc.pa.sched[i] = v.plan.sched[i];
    pc.pa.n_sched[i] = v.plan.n_sched[i];
    pc.pa.n_slices[i] = v.plan.n_slices[i];
  }
  pc.pa.max_tiles = v.plan.max_tiles;
  pc.pa.sync = v.plan.sync;
  pc.ri = v.ri;
  pc.x = (const uint16_t*)x;
  pc.xq = v.xq;
  pc.sx = v.sx;
  pc.gpr = shape->d_model / 128;
  pc.n_rows = v.xq ? shape->T : 0;
  pc.k = shape->top_k;
  return hip_status(moe::launch_route(R, (hipStream_t)stream));
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (validate_shape(shape) != MOE_OK) return 0;
  return layout(*shape).total;
}

size_t moe_plan_bytes(const moe_shape* shape) {
  if (validate_shape(shape) != MOE_OK) return 0;
  return plan_layout(*shape).total;
}

int moe_route(const moe_shape* shape, const moe_weights* w, const void* x, const moe_routing* out, void* ws,
              size_t ws_bytes, void* stream) {
  return route_common(shape, w, x, nullptr, out, ws, ws_bytes, stream);
}

int moe_route_forced(const moe_shape* shape, const moe_weights* w, const void* x, const int32_t* forced_idx,
                     const moe_routing* out, void* ws, size_t ws_bytes, void* stream) {
  if (!forced_idx) return MOE_ERR_INVALID_ARG;
  return route_common(shape, w, x, forced_idx, out, ws, ws_bytes, stream);
}

size_t moe_router_planes_bytes(int32_t n_experts, int32_t d_model) {
  if (n_experts < 1 || n_experts > 512 || d_model < 128 || d_model % 128 != 0) return 0;
  return moe::router_planes_bytes(d_model, n_experts);
}

int moe_pack_router(int32_t n_experts, int32_t d_model, const float* w_router, void* planes, void* stream) {
  if (moe_router_planes_bytes(n_experts, d_model) == 0 || !w_router || !planes) return MOE_ERR_INVALID_ARG;
  if (misaligned(w_router) || misaligned(planes)) return MOE_ERR_INVALID_ARG;
  const uintptr_t a = (uintptr_t)w_router, b = (uintptr_t)planes;
  const size_t na = (size_t)n_experts * d_model * 4, nb = moe_router_planes_bytes(n_experts, d_model);
  if (a < b + nb && b < a + na) return MOE_ERR_INVALID_ARG;  // overlapping buffers
  return hip_status(moe::launch_pack_router(w_router, planes, d_model, n_experts, (hipStream_t)stream));
}

int moe_forward(const moe_shape* shape, const moe_weights* w, const void* x, const moe_routing* r, void* y, void* ws,
                size_t ws_bytes, void* stream) {
  return moe_forward_stages(shape, w, x, r, y, ws, ws_bytes, MOE_STAGE_ALL, nullptr, stream);
}

}  // extern "C"

namespace {

// moe_forward_stages and moe_forward_noalloc.  noalloc: the forward's segments
// live in this device's `scratch` (ws and ws_bytes are ignored).
int forward_common(const moe_shape* shape, const moe_weights* w, const void* x, const moe_routing* r, void* y,
                   void* ws, size_t ws_bytes, bool noalloc, uint32_t stages, void* const* events, void* stream) {
  if (stages & ~(uint32_t)(MOE_STAGE_ALL | MOE_FORWARD_TEST_WAIT_TIMEOUT)) return MOE_ERR_INVALID_ARG;
  const bool test_timeout = stages & MOE_FORWARD_TEST_WAIT_TIMEOUT;
  int rc = validate_shape(shape);
  if (rc != MOE_OK) return rc;
  if (!w || !x || !y || !r || !r->topk_idx || !r->topk_w || !r->counts || !r->offsets || !r->perm || !r->plan)
    return MOE_ERR_INVALID_ARG;
  if (misaligned(x) || misaligned(y)) return MOE_ERR_INVALID_ARG;
  const bool fp8 = shape->w_dtype == MOE_FP8E4M3_B128;                  // activations quantised
  const bool scaled = fp8 || shape->w_dtype == MOE_FP8E4M3_B128_A16 ||  // block-scaled FP8 weights
                      shape->w_dtype == MOE_U4_G64;                       // or 4-bit group parameters
  const bool has_shared = shape->d_ffn_shared > 0;
  if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
  if (scaled && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARG;
  if (has_shared && (!w->sh_gate || !w->sh_up || !w->sh_down)) return MOE_ERR_INVALID_ARG;
  if (has_shared && scaled && (!w->ss_gate || !w->ss_up || !w->ss_down)) return MOE_ERR_INVALID_ARG;
  if (misaligned(w->w_gate) || misaligned(w->w_up) || misaligned(w->w_down)) return MOE_ERR_INVALID_ARG;
  if (has_shared && (misaligned(w->sh_gate) || misaligned(w->sh_up) || misaligned(w->sh_down)))
    return MOE_ERR_INVALID_ARG;
  if (shape->T == 0) return MOE_OK;
  const Layout L = layout(*shape, noalloc);
  if (noalloc) {
    if (L.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_LIMIT;
    if (r->plan_bytes < plan_layout(*shape).total) return MOE_ERR_WORKSPACE;
    const int src = device_scratch(&ws);
    if (src != MOE_OK) return src;
  } else {
    if (!ws) return MOE_ERR_INVALID_ARG;
    if (ws_bytes < L.total || r->plan_bytes < plan_layout(*shape).total) return MOE_ERR_WORKSPACE;
  }

  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  const int T = shape->T, d = shape->d_model, E = shape->n_experts, k = shape->top_k, P = T * k;

  ExpertArgs a;
  a.sched = nullptr;
  a.offsets = r->offsets;
  a.perm = r->perm;
  a.topk_w = r->topk_w;
  a.T = T;
  a.d = d;
  a.E = E;
  a.k = k;
  a.F = shape->d_ffn;
  a.Fs = shape->d_ffn_shared;
  a.P = P;
  a.hstride = a.F > a.Fs ? a.F : a.Fs;
  a.w_tiled = shape->w_layout == MOE_LAYOUT_TILED;
  const PlanView v = plan_view(*shape, r->plan);
  a.xa = fp8 ? (const void*)v.xq : x;
  a.sxa = v.sx;
  a.wg = w->w_gate;
  a.wu = w->w_up;
  a.wd = w->w_down;
  a.sg = (const float*)w->s_gate;
  a.su = (const float*)w->s_up;
  a.sd = (const float*)w->s_down;
  a.shg = w->sh_gate;
  a.shu = w->sh_up;
  a.shd = w->sh_down;
  a.ssg = (const float*)w->ss_gate;
  a.ssu = (const float*)w->ss_up;
  a.ssd = (const float*)w->ss_down;
  a.h = base + L.h;
  a.sh = (float*)(base + L.sh);
  a.part = (float*)(base + L.part);
  a.ri = v.ri;

  hipError_t e = hipSuccess;
  auto mark = [&](int i) {
    if (events && e == hipSuccess) e = hipEventRecord((hipEvent_t)events[i], st);
  };
  const moe::Plan& plan = v.plan;
  const int Fmax = a.F > a.Fs ? a.F : a.Fs;
  const bool fused = (stages & MOE_STAGE_GATE_UP) && (stages & MOE_STAGE_DOWN) && r->status &&
                     moe::experts_fusable(shape->w_dtype, plan, Fmax, d);
  mark(0);
  if (fused) {  // both projections in one launch: events 1 and 2 mark its end
    e = moe::launch_experts_fused(a, shape->w_dtype, plan, r->status, r->forward_status, test_timeout, st);
    mark(1);
    mark(2);
  } else if (stages & MOE_STAGE_GATE_UP) {
    e = moe::launch_gateup(a, shape->w_dtype, plan, st);
    mark(1);
  }
  if (e == hipSuccess && !fused && (stages & MOE_STAGE_DOWN)) {
    e = moe::launch_down(a, shape->w_dtype, plan, st);
    mark(2);
  }
  if (e == hipSuccess && (stages & MOE_STAGE_COMBINE)) {
    e = moe::launch_combine(a.part, r->topk_idx, T, k, d, E, P, has_shared, y, shape->act_dtype == MOE_BF16, st);
    mark(3);
  }
  return hip_status(e);
}

}  // namespace

extern "C" {

int moe_forward_stages(const moe_shape* shape, const moe_weights* w, const void* x, const moe_routing* r, void* y,
                       void* ws, size_t ws_bytes, uint32_t stages, void* const* events, void* stream) {
  return forward_common(shape, w, x, r, y, ws, ws_bytes, false, stages, events, stream);
}

int moe_forward_noalloc(const moe_shape* shape, const moe_weights* w, const void* x, const moe_routing* r, void* y,
                        void* stream) {
  return forward_common(shape, w, x, r, y, nullptr, 0, true, MOE_STAGE_ALL, nullptr, stream);
}

int moe_quantize_rows(int64_t n_rows, int32_t n_cols, int32_t act_dtype, const void* in, uint8_t* codes,
                      float* scales, void* stream) {
  if (n_rows < 0 || n_cols <= 0 || n_cols % 128 || (act_dtype != MOE_F32 && act_dtype != MOE_BF16))
    return n_cols > 0 && n_cols % 128 ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG;
  if (n_rows == 0) return MOE_OK;
  if (!in || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (misaligned(in) || misaligned(codes)) return MOE_ERR_INVALID_ARG;
  if ((n_rows + 3) / 4 * 256 > (int64_t)UINT_MAX) return MOE_ERR_UNSUPPORTED;  // one wave per row, 32-bit grid
  return hip_status(moe::launch_quantize_rows(in, act_dtype == MOE_BF16, n_rows, n_cols, codes, scales,
                                              (hipStream_t)stream));
}

int moe_pack_weights(int64_t n_mats, int32_t rows, int32_t row_bytes, const void* in, void* out, void* stream) {
  if (n_mats < 0 || rows <= 0 || row_bytes <= 0) return MOE_ERR_INVALID_ARG;
  if (rows % 16 || row_bytes % 128) return MOE_ERR_UNSUPPORTED;
  if (n_mats == 0) return MOE_OK;
  if (!in || !out) return MOE_ERR_INVALID_ARG;
  const int64_t bytes = n_mats * rows * (int64_t)row_bytes;
  const char *i0 = (const char*)in, *o0 = (const char*)out;
  if (i0 < o0 + bytes && o0 < i0 + bytes) return MOE_ERR_INVALID_ARG;  // overlap
  if (bytes / 16 / 256 >= (int64_t)UINT_MAX) return MOE_ERR_UNSUPPORTED;
  return hip_status(moe::launch_pack_weights(n_mats, rows, row_bytes, in, out, (hipStream_t)stream));
}

int moe_pack_weights_u4(int64_t n_mats, int32_t rows, int32_t cols, const void* codes, const uint16_t* scales,
                        const uint16_t* biases, void* codes_out, void* params_out, void* stream) {
  if (n_mats < 0 || rows <= 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (rows % 16 || cols % 128) return MOE_ERR_UNSUPPORTED;
  if (n_mats == 0) return MOE_OK;
  if (!codes || !scales || !biases || !codes_out || !params_out) return MOE_ERR_INVALID_ARG;
  const int64_t cbytes = n_mats * rows * (int64_t)cols / 2, pbytes = n_mats * rows * (int64_t)(cols / 64) * 4;
  auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
    const char *a0 = (const char*)a, *b0 = (const char*)b;
    return a0 < b0 + nb && b0 < a0 + na;
  };
  if (overlap(codes, cbytes, codes_out, cbytes) || overlap(codes_out, cbytes, params_out, pbytes) ||
      overlap(scales, pbytes / 2, params_out, pbytes) || overlap(biases, pbytes / 2, params_out, pbytes))
    return MOE_ERR_INVALID_ARG;
  if (cbytes / 4 / 256 >= (int64_t)UINT_MAX) return MOE_ERR_UNSUPPORTED;
  return hip_status(
      moe::launch_pack_u4(n_mats, rows, cols, codes, scales, biases, codes_out, params_out, (hipStream_t)stream));
}

size_t moe_route_compare_workspace_bytes(int32_t T) { return T < 0 ? 0 : moe::route_compare_ws_bytes(T); }

int moe_route_compare(int32_t T, int32_t E, int32_t k, const float* logits, const float* ref_logits,
                      const float* sel_bias, const int32_t* idx, const int32_t* ref_idx, float* gap, double* sigma,
                      int32_t* n_disagree, float* max_gap, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (k > moe::kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (!logits || !ref_logits || !idx || !ref_idx || !gap || !sigma || !n_disagree || !max_gap)
    return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!ws) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < moe::route_compare_ws_bytes(T)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route_compare(T, E, k, logits, ref_logits, sel_bias, idx, ref_idx, gap, sigma,
                                              n_disagree, max_gap, ws, (hipStream_t)stream));
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer or invalid size";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or dtype combination not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP kernel launch failed";
    case MOE_ERR_FORCED_INDEX: return "MOE_ERR_FORCED_INDEX: a forced expert id was outside [0, n_experts)";
    case MOE_ERR_DEVICE_SYNC: return "MOE_ERR_DEVICE_SYNC: a forward block's wait for another block timed out";
    case MOE_ERR_SCRATCH_LIMIT:
      return "MOE_ERR_SCRATCH_LIMIT: the shape needs more scratch than moe_forward_noalloc's static buffer holds";
    default: return "unknown moe status";
  }
}

}  // extern "C"
