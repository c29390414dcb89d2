/*
 * lola.h -- C ABI of the LoLA layer hot path on AMD Instinct MI355X (gfx950).
 *
 * LoLA (low-rank linear attention with sparse caching) splits the past
 * key/value pairs of every (sequence, KV head) into three memories: a
 * sliding window and a sparse cache, both read with exact softmax, and the
 * recurrent state (H, s) of linear attention with the feature map
 *   phi(x) = [softmax(W x); softmax(-W x)]
 * (paper abstract "LoLA: Low-Rank Linear Attention With Sparse Caching";
 * technical summary on gist.science, section "Methodologie: LoLA").
 *
 * At every update interval the pairs leaving the window and the cached pairs
 * are scored with the self-recall error
 *   SRE(k, v | H, s) = || H^T phi(k) / (s . phi(k)) - v ||^2
 * (summary, section "Het Self-Recall Error (SRE) Mechanisme", SRE equation);
 * the highest stay in the cache, the rest are folded into the state by outer
 * products H += phi(k) v^T, s += phi(k), and each query's output combines the
 * linear, cache and window attention (summary, section "Inferentiestrategie",
 * steps 1-4).
 *
 * Readings this library implements where the pages leave a step open:
 *   - each query reads the memories as they stand at the start of its
 *     interval; keys that leave the window earlier in the same interval are
 *     read linearly (weight phi(q).phi(k)) until the interval end manages them;
 *   - the three parts share one softmax denominator with unit weights;
 *   - scores use the interval-start state; an empty state predicts 0;
 *   - keep order is (SRE descending, position ascending); if all candidates
 *     fit, all are kept;
 *   - the window holds the last `window` tokens including the current one;
 *   - softmax scale on q.k is 1/sqrt(head_dim) unless given; none inside phi.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned and densely packed in the layouts stated.  The library never
 *     allocates, frees or keeps a pointer between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Calls only enqueue work on it and never wait for the device, except
 *     lola_check_state, which is documented as synchronous.
 *   - io dtype (q, k, v, out, cached and windowed keys/values) is fp32 or
 *     bf16; H, s and W are always fp32.
 *   - Errors are returned as lola_status before anything is enqueued;
 *     a failed HIP launch returns LOLA_ERR_HIP.  Nothing aborts or prints.
 *   - One state buffer must not be used by two calls at once (on any
 *     streams); distinct state buffers are independent.
 *   - Supported shapes: head_dim 64 or 128; feat_half 32 or 64;
 *     n_q_heads / n_kv_heads <= 16; window <= 8192; cache_cap <= 1024;
 *     chunk <= 256; positions below 2^31 per sequence.
 */
#ifndef LOLA_H
#define LOLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LOLA_OK = 0,
    LOLA_ERR_INVALID_ARG = -1, /* null / misaligned pointer, bad count or size */
    LOLA_ERR_UNSUPPORTED = -2, /* shape or dtype outside the supported set */
    LOLA_ERR_BAD_STATE = -3,   /* state header does not match the config */
    LOLA_ERR_WORKSPACE = -4,   /* workspace smaller than lola_prefill_workspace_bytes */
    LOLA_ERR_HIP = -5          /* a HIP runtime call or launch failed */
} lola_status;

typedef enum { LOLA_F32 = 0, LOLA_BF16 = 1 } lola_dtype;

typedef struct {
    int32_t n_q_heads;     /* Hq; a multiple of n_kv_heads (query head h reads KV head h / (Hq/Hkv)) */
    int32_t n_kv_heads;    /* Hkv */
    int32_t head_dim;      /* D */
    int32_t feat_half;     /* rows of W; feature dimension F = 2 * feat_half */
    int32_t window;        /* w >= 0: last-w softmax window (0: none) */
    int32_t cache_cap;     /* C >= 0: sparse cache capacity per (sequence, KV head) */
    int32_t chunk;         /* L >= 1: update interval length of lola_prefill_chunk */
    int32_t io_dtype;      /* lola_dtype */
    float softmax_scale;   /* tau on q.k; <= 0 selects 1/sqrt(head_dim) */
} lola_config;

/* Bytes of the state buffer for `batch` sequences (header, tokens seen, W,
 * and per (sequence, KV head): H [F][D] f32, s [F] f32, cache positions,
 * window ring and cache keys/values, and for bf16 io the feature rows of the
 * cached keys).  0 if the config is not supported. */
size_t lola_state_bytes(const lola_config* cfg, int32_t batch);

/* Bytes of scratch that lola_prefill_chunk needs for up to `max_tokens`
 * tokens per call (feature rows, interval-start snapshots of H, s and the
 * cache, copies of the window and cache at the call start).  0 if invalid. */
size_t lola_prefill_workspace_bytes(const lola_config* cfg, int32_t batch, int32_t max_tokens);

/* Initialise `state` (device, lola_state_bytes) for `batch` empty sequences:
 * header, tokens seen = 0, H = 0, s = 0, empty cache and window.
 * W: device [n_kv_heads][feat_half][head_dim] f32, copied into the state. */
lola_status lola_init_state(const lola_config* cfg, int32_t batch, const float* W, void* state,
                            void* stream);

/* Advance every sequence by n_tokens (> 0) tokens: positions
 * [t0, t0 + n_tokens) are processed as consecutive update intervals of
 * cfg->chunk tokens (the last may be shorter), each call starting its own
 * interval grid at t0.  Per interval: outputs of its queries from the
 * interval-start memories, then SRE scoring of leaving + cached pairs, top-C
 * keep, fold of the rest, window update.
 *   q   [batch][n_tokens][n_q_heads][head_dim]  io dtype
 *   k,v [batch][n_tokens][n_kv_heads][head_dim] io dtype
 *   out [batch][n_tokens][n_q_heads][head_dim]  io dtype (written)
 *   workspace: device scratch of at least
 *              lola_prefill_workspace_bytes(cfg, batch, n_tokens) bytes. */
lola_status lola_prefill_chunk(const lola_config* cfg, void* state, int32_t batch, int32_t n_tokens,
                               const void* q, const void* k, const void* v, void* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* lola_prefill_chunk that also records three or four caller-created
 * hipEvent_t (passed as void*) on `stream`: events[0] before the first
 * launch, events[1] after the feature-row prologue, events[2] after the
 * interval scan, events[3] after the output pass.  Any entry may be NULL.
 * Same results as lola_prefill_chunk; meant for per-kernel timing. */
lola_status lola_prefill_chunk_timed(const lola_config* cfg, void* state, int32_t batch, int32_t n_tokens,
                                     const void* q, const void* k, const void* v, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream,
                                     void* const* events);

/* lola_prefill_chunk with a token count per sequence, for batches whose
 * sequences advance by different amounts in one call (prefill chunks of
 * several lengths, single decode tokens, idle sequences).  The method runs
 * independently per sequence (each (sequence, KV head) pair owns its window,
 * cache and linear state; LoLA summary, "Methodologie: LoLA"), so sequence b
 * gets exactly the result of lola_prefill_chunk over its own n_tokens[b]
 * tokens, with its update intervals counted from its own start.
 *   n_tokens: device [batch] int32, 4-byte aligned, read by the kernels; each
 *             entry is clamped to [0, max_tokens] (0 leaves the sequence,
 *             including its token count, unchanged)
 *   q, k, v, out: laid out as for lola_prefill_chunk with max_tokens rows per
 *             sequence; sequence b reads and writes its first n_tokens[b] rows,
 *             the other rows of out are not written
 *   workspace: at least lola_prefill_workspace_bytes(cfg, batch, max_tokens).
 * Host-side checks as for lola_prefill_chunk (max_tokens > 0), plus
 * LOLA_ERR_INVALID_ARG for a NULL or misaligned n_tokens. */
lola_status lola_prefill_ragged(const lola_config* cfg, void* state, int32_t batch, int32_t max_tokens,
                                const int32_t* n_tokens, const void* q, const void* k, const void* v,
                                void* out, void* workspace, size_t workspace_bytes, void* stream);

/* One token for every sequence: identical in result to
 * lola_prefill_chunk(n_tokens = 1) (a one-token interval), in one fused launch
 * that needs no workspace.
 *   q [batch][n_q_heads][head_dim], k, v [batch][n_kv_heads][head_dim],
 *   out [batch][n_q_heads][head_dim], all io dtype. */
lola_status lola_decode_step(const lola_config* cfg, void* state, int32_t batch, const void* q,
                             const void* k, const void* v, void* out, void* stream);

/* Copy the memories out of `state` into caller device buffers (any output
 * may be NULL).  Cache entries are written in ascending position order.
 *   count [batch][n_kv_heads] int32       entries held
 *   pos   [batch][n_kv_heads][cache_cap]  int64, ascending, -1 padded
 *   k_out, v_out [batch][n_kv_heads][cache_cap][head_dim] io dtype, 0 padded
 *   H_out [batch][n_kv_heads][F][head_dim] f32,  s_out [batch][n_kv_heads][F] f32
 *   tokens_seen [batch] int64
 * Valid once the stream has reached this call. */
lola_status lola_read_cache(const lola_config* cfg, const void* state, int32_t batch, int32_t* count,
                            int64_t* pos, void* k_out, void* v_out, float* H_out, float* s_out,
                            int64_t* tokens_seen, void* stream);

/* SYNCHRONOUS: waits for `stream`, then reads the state header and returns
 * LOLA_OK if it was written by lola_init_state for this config and batch and
 * no call has marked it faulted, LOLA_ERR_BAD_STATE otherwise.  With bf16 io
 * and few enough (sequence, KV head) chains to be resident together, the
 * interval scan of lola_prefill_chunk spreads each chain over head_dim/16
 * workgroups (a cooperative launch) that wait for one another once per
 * interval; a wait that does not end within a fixed bound marks the state
 * faulted instead of hanging. */
lola_status lola_check_state(const lola_config* cfg, const void* state, int32_t batch, void* stream);

/* Static text for a status code (never NULL). */
const char* lola_status_string(lola_status status);

#ifdef __cplusplus
}
#endif

#endif /* LOLA_H */
