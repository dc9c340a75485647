/*
 * moe_attn.h - C ABI of the attention ops next to the mixture-of-experts layer
 * (MI355X, gfx950): rotary position encoding, and causal attention over a
 * sliding window or the whole context.
 *
 * Sources, cited by page title and section:
 *   [port]  "We Ported Aleph Alpha's Kolibri to a MacBook. Our Own Gate Said No."
 *           (localfirstai.eu, 5 October 2026)
 *   [bench] "We Stopped the Kolibri Benchmark Before Scoring One Answer"
 *           (localfirstai.eu, 9 October 2026)
 *
 * [port] "The gate": forty layers attend over a sliding window of 513 tokens
 * and mark position with rotary position encoding; every fifth layer attends
 * over the whole context with no positional encoding (the same layout in
 * [bench] "The pilot that ran out of buffers, not memory").  [port] "Taking it
 * apart", part 2: each pair of dimensions of a query or key is rotated by the
 * token's position times a fixed frequency, textbook 1/theta^(2j/D).
 *
 * Conventions as in moe.h: device pointers, row-major, caller-owned buffers,
 * calls enqueue on `stream` without synchronising, host-detectable errors
 * return a negative status and enqueue nothing, T == 0 enqueues nothing.
 * Tensors are bf16 (bit patterns, 2 bytes per element).
 */
#ifndef MOE_ATTN_H
#define MOE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_ATTN_OK = 0,
  MOE_ATTN_ERR_INVALID_ARG = -1, /* null pointer, negative or inconsistent size */
  MOE_ATTN_ERR_UNSUPPORTED = -2, /* valid but unsupported (head_dim other than 128, ...) */
  MOE_ATTN_ERR_WORKSPACE = -3,   /* ws_bytes below moe_attn_workspace_bytes() */
  MOE_ATTN_ERR_HIP = -4          /* a HIP launch failed */
};

typedef struct {
  int32_t n_q_heads;  /* Hq */
  int32_t n_kv_heads; /* Hkv; divides Hq, and Hq/Hkv divides 64.  Query head h
                         reads key/value head h / (Hq/Hkv) */
  int32_t head_dim;   /* D; 128 */
  int32_t window;     /* W > 0: a query at position p attends keys p-W+1 .. p
                         (the pages' sliding layers: 513); 0: every key <= p */
} moe_attn_shape;

/* Rotary position encoding, in place.  x [T, n_heads, head_dim] bf16; token t
 * sits at position pos0 + t.  For j < head_dim/2 the pair (x_j, x_{j+D/2}) is
 * rotated by the angle (pos0 + t) / theta^(2j/D):
 *   x_j' = x_j cos - x_{j+D/2} sin,  x_{j+D/2}' = x_j sin + x_{j+D/2} cos,
 * the angle formed and reduced modulo 2 pi in double, the rotation in fp32,
 * rounded once to bf16 (nearest, ties to even); head_dim <= 1024.  Apply it
 * to new queries and keys before they enter moe_attention (keys are cached
 * rotated); whole-context layers without positional encoding skip it. */
int moe_rope(int32_t T, int32_t n_heads, int32_t head_dim, int32_t pos0, float theta, void *x, void *stream);

/* Workspace bytes moe_attention needs for this call shape (0 when none or when
 * the shape is invalid).  Short query batches split each row's keys over
 * several blocks and need room for the partial results. */
size_t moe_attn_workspace_bytes(const moe_attn_shape *s, int32_t Tq, int32_t Tk, int32_t q_pos0);

/* Causal attention of Tq queries against a cache of Tk keys and values.
 * q [Tq, Hq, D], k and v [Tk, Hkv, D] (the cache: key j at position j), o
 * [Tq, Hq, D], all bf16.  Query i sits at position q_pos0 + i; needs
 * q_pos0 + Tq <= Tk.  o = softmax(q k^T / sqrt(D)) v over the keys the query
 * attends (see moe_attn_shape.window), scores and softmax in fp32, the
 * probabilities split into two bf16 parts (high, and the remainder) for the
 * product with v, o rounded to bf16. */
int moe_attention(const moe_attn_shape *s, int32_t Tq, int32_t Tk, int32_t q_pos0, const void *q, const void *k,
                  const void *v, void *o, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ATTN_H */
