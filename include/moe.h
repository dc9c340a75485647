/*
 * moe.h - C ABI of the MI355X (gfx950) mixture-of-experts layer forward pass.
 *
 * One layer: a float32 router scores every expert for every token; each token
 * goes to its top-k experts (free routing, selection by logit plus an optional
 * per-expert selection bias, lowest expert index on ties) or to experts the
 * caller recorded earlier (forced routing); the routed experts and one shared
 * expert run a SwiGLU FFN; a fixed-order weighted sum combines their outputs.
 *
 * Sources, cited by page title and section:
 *   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
 *           (localfirstai.eu, 5 October 2026)
 *   [bench] "We Stopped the Kolibri Benchmark Before Scoring One Answer"
 *           (localfirstai.eu, 9 October 2026)
 *   [cache] "Kolibri-1 CPU dequant cache" (vllm.cpp pull request 3488)
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (HBM of the current HIP device),
 *     row-major, densely packed, each 16-byte aligned (the kernels move 16 bytes
 *     per lane; hipMalloc and torch allocations are 256-byte aligned, and every
 *     row width the shapes allow keeps later rows aligned).  Buffers that are not
 *     16-byte aligned return MOE_ERR_INVALID_ARG where the call checks them (the
 *     activation rows and outputs of moe_route, moe_forward and
 *     moe_quantize_rows); for the others behaviour is undefined.  The caller allocates and owns every buffer,
 *     including the workspace; the library never allocates or frees memory and
 *     keeps no state between calls (calls are reentrant).
 *   - Calls enqueue kernels on `stream` (a hipStream_t; NULL = the default
 *     stream) and return without synchronising.  No device-to-host copy is made.
 *   - Errors the host can detect return a negative moe_status and enqueue
 *     nothing.  A failed kernel launch returns MOE_ERR_HIP.  Errors only the
 *     device can see (invalid forced expert ids) are written to the device
 *     status word `moe_routing.status`, which the caller reads after its own
 *     synchronisation.
 *   - T == 0 returns MOE_OK and enqueues nothing.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null pointer, negative or inconsistent size */
  MOE_ERR_UNSUPPORTED = -2,  /* valid but unsupported shape or dtype combination */
  MOE_ERR_WORKSPACE = -3,    /* ws_bytes below moe_workspace_bytes(), or moe_routing.plan_bytes
                                below moe_plan_bytes() */
  MOE_ERR_HIP = -4,          /* a HIP launch failed */
  MOE_ERR_FORCED_INDEX = -5, /* (device status) a forced expert id was outside [0, E) */
  MOE_ERR_DEVICE_SYNC = -6,  /* (device status) inside moe_forward, a block's bounded wait for
                                another block's results ran out; y is not valid */
  MOE_ERR_SCRATCH_LIMIT = -7 /* moe_forward_noalloc: the shape needs more than
                                MOE_NOALLOC_SCRATCH_BYTES of scratch */
} moe_status;

typedef enum {
  MOE_F32 = 0,           /* float32 */
  MOE_BF16 = 1,          /* bfloat16 */
  MOE_FP8E4M3_B128 = 2,  /* OCP FP8 E4M3 codes, value = decode(code) * scale of its
                            128 x 128 block (fp32 scales); weights only.  The activations
                            entering each projection are quantised to E4M3 (see moe_forward) */
  MOE_FP8E4M3_B128_A16 = 3, /* the same weights as W8A16: activations enter both
                              projections in bf16, unquantised, and h stays bf16
                              ([cache]: the CPU runtime decodes the FP8 weights for its
                              matmuls on bf16 activations); weights only */
  MOE_U4_G64 = 4           /* 4-bit affine groups: per row and group of 64 consecutive
                              columns a bf16 scale and bias, value = scale * q + bias
                              with q the unsigned 4-bit code (the 4-bit build of [bench]
                              "The gate, forced", read as MLX's default group
                              quantisation); activations enter in bf16, unquantised,
                              and h stays bf16; weights only, MOE_LAYOUT_TILED only */
} moe_dtype;

/* Supported (act_dtype, w_dtype) pairs: (F32, F32), (BF16, BF16), (BF16, FP8E4M3_B128),
 * (BF16, FP8E4M3_B128_A16), (BF16, U4_G64).
 * Limits: 1 <= top_k <= 8, top_k <= n_experts <= 512, d_model and d_ffn multiples
 * of 128, d_ffn_shared 0 (no shared expert) or a multiple of 128, T * top_k < 2^31.
 * The expert kernels hold one 16-row tile's activation rows (d_model wide) and h
 * rows (max(d_ffn, d_ffn_shared) wide) in the 160 KB of LDS of one workgroup, which
 * bounds the widths: d_model <= 4608 for FP8E4M3_B128, FP8E4M3_B128_A16 and U4_G64
 * weights, <= 4736 for BF16, <= 2560 for F32; d_ffn and d_ffn_shared <= 4096, and
 * <= 2560 for F32.  Wider shapes return MOE_ERR_UNSUPPORTED. */
/* Layouts of the expert weight matrices (moe_shape.w_layout). */
typedef enum {
  MOE_LAYOUT_ROWMAJOR = 0,   /* [rows][cols] row-major, as documented per tensor */
  MOE_LAYOUT_TILED = 1       /* the same bytes regrouped by moe_pack_weights into 2 KB
                                tiles of 16 rows x 128 bytes (bf16: 64 columns); 4-bit
                                weights: the codes and group parameters as
                                moe_pack_weights_u4 writes them */
} moe_layout;

typedef struct {
  int32_t T;             /* tokens in this call */
  int32_t d_model;       /* d */
  int32_t n_experts;     /* E (routed experts) */
  int32_t top_k;         /* k */
  int32_t d_ffn;         /* F, routed expert FFN width */
  int32_t d_ffn_shared;  /* Fs, shared expert FFN width; 0 = no shared expert */
  int32_t act_dtype;     /* moe_dtype of x and y: MOE_F32 or MOE_BF16 */
  int32_t w_dtype;       /* moe_dtype of the expert weights */
  int32_t w_layout;      /* moe_layout of w_gate, w_up, w_down, sh_gate, sh_up, sh_down;
                            MOE_LAYOUT_TILED needs w_dtype BF16, an FP8 one or U4_G64;
                            U4_G64 needs MOE_LAYOUT_TILED */
} moe_shape;

/* Layer weights.  Expert matrices are (out, in) row-major and stacked by expert.
 * Scales are required for MOE_FP8E4M3_B128 and MOE_FP8E4M3_B128_A16 (fp32 block
 * scales, shapes below) and for MOE_U4_G64 (each s_* / ss_* then points to the
 * group parameters moe_pack_weights_u4 wrote for that matrix stack, 4 bytes per
 * row and 64-column group, and w_* / sh_* to its packed codes), and ignored
 * otherwise.
 *   [port] "The gate": a router scores the experts for every token and a shared
 *   expert serves every token; part 1 of "Taking it apart": selection uses the
 *   router score plus a per-expert selection bias; part 3: the router runs in
 *   float32.  [cache], first paragraph: the expert weights are FP8 and must be
 *   decoded for compute. */
typedef struct {
  const float *w_router;  /* [E, d] fp32 */
  const float *sel_bias;  /* [E] fp32, or NULL; enters expert selection only */
  const void *w_gate;     /* [E, F, d] */
  const void *w_up;       /* [E, F, d] */
  const void *w_down;     /* [E, d, F] */
  const void *s_gate;     /* [E, F/128, d/128] block scales */
  const void *s_up;       /* [E, F/128, d/128] */
  const void *s_down;     /* [E, d/128, F/128] */
  const void *sh_gate;    /* shared expert [Fs, d] (ignored when Fs == 0) */
  const void *sh_up;      /* [Fs, d] */
  const void *sh_down;    /* [d, Fs] */
  const void *ss_gate;    /* [Fs/128, d/128] */
  const void *ss_up;      /* [Fs/128, d/128] */
  const void *ss_down;    /* [d/128, Fs/128] */
  const void *w_router_planes; /* w_router packed by moe_pack_router, or NULL.  Optional: when
                            given, routing calls with bf16 activations and more than 1024
                            (token, slot) pairs read the router weights from it instead of
                            splitting w_router in every call; the logits are the same bit
                            for bit.  It must hold the current w_router (16-byte aligned). */
} moe_weights;

/* Routing results (written by moe_route / moe_route_forced, read by moe_forward).
 * Pairs are numbered p = t * k + j (token t, slot j). */
typedef struct {
  float *logits;       /* [T, E] fp32 router logits, or NULL (then not written) */
  int32_t *topk_idx;   /* [T, k] expert ids; free: descending selection score;
                          forced: the caller's order; -1 marks an invalid forced id */
  float *topk_w;       /* [T, k] routing weights: softmax over the chosen experts'
                          (unbiased) logits; 0 for an invalid slot */
  int32_t *counts;     /* [E] pairs per expert */
  int32_t *offsets;    /* [E + 1] exclusive prefix sum of counts */
  int32_t *perm;       /* [T * k] perm[q] = p: pairs sorted by expert, ascending p
                          within an expert; entries past offsets[E] are -1 */
  int32_t *inv_perm;   /* [T * k] inv_perm[p] = q, or -1 for an invalid pair */
  int32_t *status;     /* [1] device status word: MOE_OK, MOE_ERR_FORCED_INDEX (routing)
                          or MOE_ERR_DEVICE_SYNC (forward); every routing call resets it */
  void *plan;          /* at least moe_plan_bytes() bytes: the dispatch plan the routing
                          call writes for moe_forward (expert-kernel block schedules,
                          per-row token/weight, with FP8 weights the activations
                          as E4M3 codes with per-(token, 128) scales, and per-tile
                          counters the forward's blocks synchronise on); opaque */
  size_t plan_bytes;   /* bytes the caller allocated at plan; fewer than moe_plan_bytes()
                          for the call's shape return MOE_ERR_WORKSPACE before any launch */
  int32_t *forward_status; /* [1] device word, or NULL.  Sticky: moe_forward writes
                          MOE_ERR_DEVICE_SYNC here (besides *status) when a bounded wait
                          runs out, and no library call ever clears it, so one read
                          after any number of route/forward calls tells whether one
                          failed.  The caller zeroes it. */
} moe_routing;

/* Workspace bytes needed by moe_route, moe_route_forced and moe_forward for this
 * shape (one size serves all three).  Returns 0 for an invalid shape.  The
 * workspace carries nothing from one call to the next. */
size_t moe_workspace_bytes(const moe_shape *shape);

/* Bytes of moe_routing.plan for this shape.  Returns 0 for an invalid shape. */
size_t moe_plan_bytes(const moe_shape *shape);

/* Free routing.  Router logits l = x W_r^T (fp32 accumulation); selection score
 * s = l + sel_bias (selection only); top-k of s, lowest expert index on ties;
 * weights softmax over the k chosen logits; then the dispatch: counts, offsets,
 * and the stable permutation of pairs by expert ([port] part 3 and its update:
 * the expert matmul runs over (token, expert) rows sorted by expert), and the
 * dispatch plan in out->plan (with FP8 weights it includes the activations
 * quantised as moe_quantize_rows does).  x is [T, d] in act_dtype.  Sets
 * *status = MOE_OK. */
int moe_route(const moe_shape *shape, const moe_weights *w, const void *x, const moe_routing *out,
              void *ws, size_t ws_bytes, void *stream);

/* Forced routing ([bench] "The gate, forced": recorded expert choices are
 * replayed).  forced_idx [T, k] int32 device array; ids are used as given and in
 * the given slot order (duplicates are computed literally); weights are the
 * softmax over the logits at those ids.  An id outside [0, E) sets
 * *status = MOE_ERR_FORCED_INDEX, is stored as -1 with weight 0, is not
 * dispatched, and the token's other slots are renormalised among themselves. */
int moe_route_forced(const moe_shape *shape, const moe_weights *w, const void *x, const int32_t *forced_idx,
                     const moe_routing *out, void *ws, size_t ws_bytes, void *stream);

/* Expert FFNs and combine.  For every routed pair and for the shared expert:
 * SwiGLU h = silu(W_gate x) * (W_up x), y_e = W_down h.  With MOE_FP8E4M3_B128
 * weights the activations entering each projection are quantised per token and
 * per 128-element group to E4M3 with scale amax/448 (round to nearest even,
 * saturating); with MOE_FP8E4M3_B128_A16 they enter as bf16 (h rounded to bf16).
 * With either, each 128 x 128 block's products are summed exactly in fp32 and
 * the block scales applied in fp32.  With MOE_U4_G64 x and h (rounded to bf16)
 * enter as bf16 and each weight is scale * q + bias of its (row, 64-column
 * group), summed per group in fp32 as scale * sum(x * q) + bias * sum(x).
 * Combine per token, in
 * fp32 and this order: acc = shared; acc += w_j * y_j for j = 0..k-1;
 * y = acc rounded to act_dtype (bf16: round to nearest even).
 * `r` must hold the results of moe_route / moe_route_forced for the same shape
 * and x (its plan included; logits, counts, offsets, perm and inv_perm are
 * not read).  y is [T, d] in act_dtype.  With FP8 weights (either mode) in
 * 16-row tiles the two projections run as one launch whose down blocks wait on per-tile
 * counters in the plan (reset before the launch ends): a plan serves any
 * number of forward calls, one at a time; forward calls that overlap on one
 * plan race.  If such a wait runs out (it cannot when blocks start in order),
 * *r->status and *r->forward_status (when given) become MOE_ERR_DEVICE_SYNC,
 * y is not valid, and the plan must be rebuilt by a routing call. */
int moe_forward(const moe_shape *shape, const moe_weights *w, const void *x, const moe_routing *r, void *y,
                void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: moe_forward
 * with no workspace argument.  The forward's scratch (h rows, their scales, the
 * fp32 partial outputs) lives in a static device buffer of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends; its address is looked up once per device (on that
 * device's first call), and the call itself allocates and frees nothing.
 * Scratch the shape needs, with R = T * top_k + T rows, H = max(d_ffn,
 * d_ffn_shared), h bytes hb = 1 (MOE_FP8E4M3_B128), 4 (MOE_F32), else 2, and
 * a256(n) = n rounded up to a multiple of 256:
 *   a256(R * H * hb) + a256(MOE_FP8E4M3_B128 ? R * H / 128 * 4 : 0) + a256(R * d_model * 4);
 * more than MOE_NOALLOC_SCRATCH_BYTES returns MOE_ERR_SCRATCH_LIMIT before any
 * launch (the d_model 2048, d_ffn 640, top-6 FP8 layer fits up to T = 1083).
 * Nothing in the buffer needs to start at zero.  Every call on one device
 * shares that device's buffer, which keeps the last call's contents: calls that
 * overlap on one device (other streams, other host threads) race with each
 * other.  Arguments, other errors and results are those of moe_forward with the
 * same arguments, bitwise. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_forward_noalloc(const moe_shape *shape, const moe_weights *w, const void *x, const moe_routing *r, void *y,
                        void *stream);

/* Stages of moe_forward, in launch order. */
enum {
  MOE_STAGE_GATE_UP = 1,   /* grouped gate/up projections + SwiGLU (+ h quantisation) */
  MOE_STAGE_DOWN = 2,      /* grouped down projection, times the routing weight */
  MOE_STAGE_COMBINE = 4,   /* fixed-order combine into y */
  MOE_STAGE_ALL = 7,
  /* Test hook for the error path of the one-launch expert kernel (no effect on
     other launches): every down block waits for one gate/up block more than its
     tile has, gives up after 16 polls and goes on, so the launch ends normally
     with MOE_ERR_DEVICE_SYNC in *status and *forward_status and y is not valid.
     The plan's per-tile counters may then be left non-zero: a routing call
     must rebuild the plan before the next forward. */
  MOE_FORWARD_TEST_WAIT_TIMEOUT = 0x100
};

/* moe_forward restricted to a subset of its stages (bitmask of MOE_STAGE_*, plus
 * optionally MOE_FORWARD_TEST_WAIT_TIMEOUT),
 * optionally timed.  Calling the stages one at a time, in order, on one stream
 * with the same arguments and workspace gives bitwise the result of
 * moe_forward; the intermediate results live in the workspace between the
 * calls.  `events` is NULL or an array of 4 hipEvent_t created by the caller:
 * events[0] is recorded on `stream` before the first stage and events[i] right
 * after stage i (1 = gate/up .. 3 = combine) when that stage is selected, so the
 * interval between two records spans only that stage's kernels.  When gate/up
 * and down are both selected and run as one launch (see moe_forward), events[1]
 * and events[2] are both recorded after it.  Unknown stage bits:
 * MOE_ERR_INVALID_ARG. */
int moe_forward_stages(const moe_shape *shape, const moe_weights *w, const void *x, const moe_routing *r, void *y,
                       void *ws, size_t ws_bytes, uint32_t stages, void *const *events, void *stream);

/* The activation quantisation used by moe_forward on its own: each of the n_rows
 * rows of `in` ([n_rows, n_cols], act_dtype MOE_F32 or MOE_BF16, n_cols a multiple
 * of 128) is cut into groups of 128; per group scale = amax/448 (1 for an all-zero
 * group) and codes = E4M3(v / scale), round to nearest even, saturating at 448.
 * codes [n_rows, n_cols] uint8, scales [n_rows, n_cols/128] fp32.  The pages do
 * not say how FP8 activations are formed; this is the per-token, per-128-group
 * dynamic reading. */
int moe_quantize_rows(int64_t n_rows, int32_t n_cols, int32_t act_dtype, const void *in, uint8_t *codes,
                      float *scales, void *stream);

/* Regroups n_mats row-major matrices of [rows][row_bytes] bytes (rows a multiple
 * of 16, row_bytes a multiple of 128) into MOE_LAYOUT_TILED, one matrix after the
 * other in `out` (same total size; `in` and `out` must not overlap).  Tile
 * (rt, kb) of a matrix -- rows 16*rt .. 16*rt+15, bytes 128*kb .. 128*kb+127 of
 * each -- is stored at byte 2048*(rt*(row_bytes/128) + kb); inside a tile, byte j
 * (0..15) of slot (h, l) at 1024*h + 16*l holds row 16*rt + l%16, byte
 * 128*kb + 16*(l/16) + 64*h + j.  Each 16-row tile of a matrix is then one
 * contiguous run that the expert kernels stream in full cache lines.  Pack
 * w_gate and w_up as (E, F, d*bytes), w_down as (E, d, F*bytes), the shared
 * matrices with n_mats = 1; scales, router and bias keep their layout.  This
 * is a data-layout choice of this library, not something the method needs. */
int moe_pack_weights(int64_t n_mats, int32_t rows, int32_t row_bytes, const void *in, void *out, void *stream);

/* 4-bit weights (MOE_U4_G64) into MOE_LAYOUT_TILED.  Input, per matrix of the
 * n_mats stacked [rows][cols] matrices (rows a multiple of 16, cols of 128):
 * codes [rows][cols/2] bytes, column c of a row in byte c/2, the even column in
 * the low nibble; scales and biases [rows][cols/64] bf16 (group g = columns
 * 64g .. 64g+63).  Output: codes_out (same size as codes) and params_out
 * ([rows][cols/64] x 4 bytes).  Codes: tile (rt, kb) -- rows 16*rt .. 16*rt+15,
 * columns 128*kb .. 128*kb+127 -- is 1 KB at 1024*(rt*(cols/128) + kb); its
 * 32-bit word 4*l + m holds row 16*rt + l%16 and columns 128*kb + 32*m +
 * 8*(l/16) + [0, 8), the even column 2j of those 8 in bits 4j..4j+3 and the
 * odd column 2j+1 in bits 16+4j..19+4j.  Group parameters: 8 bytes at
 * 8*(16*(rt*(cols/128) + kb) + r) for row 16*rt + r: the bf16 scale and bias of
 * group 2*kb, then those of group 2*kb + 1.  Inputs and outputs must not
 * overlap.  This regrouping is a data-layout choice of this library. */
int moe_pack_weights_u4(int64_t n_mats, int32_t rows, int32_t cols, const void *codes, const uint16_t *scales,
                        const uint16_t *biases, void *codes_out, void *params_out, void *stream);

/* Bytes of the packed router weights for E experts and d_model d (0 for an
 * invalid pair: 1 <= E <= 512, d a multiple of 128). */
size_t moe_router_planes_bytes(int32_t n_experts, int32_t d_model);
/* Packs the fp32 router weights w_router [E, d] (device) into `planes`
 * (moe_router_planes_bytes(E, d) bytes, device, 16-byte aligned, not
 * overlapping w_router), once per layer ([port] part 3 of "Taking it apart":
 * the router runs in float32).  Each weight w is split exactly into three bf16
 * terms, hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid) (round to
 * nearest even; w = hi + mid + lo), the same split the router kernels make
 * from w_router; stored in matrix-core operand order: fragment (expert tile
 * et of 16 experts, 32-deep K step ks, plane p = hi, mid, lo) is 1 KB at
 * 1024 * ((et * (d/32) + ks) * 3 + p), where the 16 bytes at 16 * l hold
 * expert 16 et + l%16 at K = 32 ks + 8 (l/16) + [0, 8) (zero past E).  A
 * layout choice of this library.  Errors: MOE_ERR_INVALID_ARG for an invalid
 * shape, a null or misaligned pointer. */
int moe_pack_router(int32_t n_experts, int32_t d_model, const float *w_router, void *planes, void *stream);
/* Routing compared as a distribution: the third part of the check [port]
 * "Taking it apart" proposes (force the routing, compare the rest closely,
 * check the routing itself as a distribution), with sigma, a layer's RMS
 * router-logit error, and disagreements measured by the reference's margin in
 * units of sigma ([bench] "The gate, forced"), counted over tokens ([port]
 * "What we couldn't explain").  Inputs (device, row-major): logits and
 * ref_logits [T, E] fp32 (the side under test and the reference), sel_bias [E]
 * fp32 or NULL (the reference's selection bias), idx and ref_idx [T, k] int32
 * (each side's chosen experts, as moe_route writes them; slot order is ignored,
 * ids outside [0, E) are ignored).  Outputs (device):
 *   *sigma = sqrt(mean over the T x E entries of (logits - ref_logits)^2),
 *            summed in double;
 *   gap[t] = -1 where the two expert sets of token t agree; otherwise the
 *            largest s[e] - s[f] over experts e only the reference chose and f
 *            only the other side chose, s = ref_logits + sel_bias (fp32, then
 *            the difference in double; 0 when no such pair exists), divided by
 *            sigma (+inf for sigma = 0 and a positive margin, 0 for both 0);
 *   *n_disagree = the number of tokens whose sets differ; *max_gap = the
 *            largest gap (-1 when none differs).
 * The disagreement rate is *n_disagree / T.  Results are bitwise repeatable.
 * ws: moe_route_compare_workspace_bytes(T) bytes.  T == 0 returns MOE_OK and
 * writes nothing.  Limits: 1 <= k <= 8, k <= E. */
size_t moe_route_compare_workspace_bytes(int32_t T);
int moe_route_compare(int32_t T, int32_t E, int32_t k, const float *logits, const float *ref_logits,
                      const float *sel_bias, const int32_t *idx, const int32_t *ref_idx, float *gap, double *sigma,
                      int32_t *n_disagree, float *max_gap, void *ws, size_t ws_bytes, void *stream);

/* Static description of a status code. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
