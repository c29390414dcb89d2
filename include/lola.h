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
 *   - The state header (magic, format version, a hash of the config and the
 *     batch, a fault word) is also tested on the device, by every kernel
 *     before it touches anything else: a state initialised for another
 *     config or batch, or one that an earlier call marked faulted, is left
 *     unchanged by lola_prefill_chunk, lola_prefill_ragged and
 *     lola_decode_step (no state byte, output row or workspace byte is
 *     written) although the call itself returns LOLA_OK, since the host
 *     never waits for the device.  lola_check_state reports such a state as
 *     LOLA_ERR_BAD_STATE.  Only the first 32 bytes of the buffer are read
 *     for the test, so a buffer sized for another config is never read or
 *     written past them.
 *   - One state buffer must not be used by two calls at once (on any
 *     streams); distinct state buffers are independent.
 *   - Supported shapes: head_dim 64 or 128; feat_half 32 or 64;
 *     n_q_heads / n_kv_heads <= 16; window <= 8192; cache_cap <= 1024;
 *     chunk <= 256; positions below 2^31 per sequence.
 *   - bf16 prefill with the default policy runs the split scan as a
 *     cooperative launch; where that launch is refused (observed: a second
 *     process on a GPU whose first process has run split scans) the call
 *     returns LOLA_ERR_HIP, and LOLA_SCAN_SPLIT=0 avoids it.
 *   - Environment: LOLA_SCAN_SPLIT=0 (read at every prefill call) makes bf16
 *     prefill use the one-workgroup-per-chain scan instead of the split scan;
 *     LOLA_TRACE=1 (read at the first launch of the process) encloses every
 *     kernel launch in a roctx range named after the kernel ("lola::prologue",
 *     "lola::scan_split", "lola::scan", "lola::output", "lola::decode"; the
 *     roctx library is opened only then, and tracing stays off if it cannot be).
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

/* How the candidates of an interval (the cached pairs and the pairs leaving the
 * window) are scored; every policy keeps the C highest scores, the older
 * position first on a tie, and folds the rest.  The method is LOLA_POLICY_SRE
 * (summary, "Inferentiestrategie", steps 1-2).  The others are the summary's
 * alternatives -- step 2's min-heap or FIFO cache structure, and the scorers its
 * contributions and ablations compare against the SRE (attention-weight
 * magnitude, softmax approximation error) -- which it names without formulas;
 * this library reads them as:
 *   LOLA_POLICY_SRE_STALE   a pair is scored by its SRE once, in the interval in
 *                           which it leaves the window; a cached pair keeps that
 *                           score (a min-heap of stale scores)
 *   LOLA_POLICY_FIFO        the score is the position: the C most recent stay
 *   LOLA_POLICY_ATTN        sum over the KV head's query heads of the softmax
 *                           weight that the interval's last query gives the
 *                           candidate among all candidates (scale softmax_scale)
 *   LOLA_POLICY_SOFTMAX_ERR sum over those heads of |that softmax weight - the
 *                           candidate's linear-attention weight
 *                           phi(q).phi(k) / sum over the candidates|
 * The policies other than LOLA_POLICY_SRE run in lola_prefill_chunk and
 * lola_prefill_ragged (any token count, so n_tokens = 1 gives the token-by-
 * token mode); lola_decode_step's fused kernel implements LOLA_POLICY_SRE only
 * and returns LOLA_ERR_UNSUPPORTED for the others. */
/* How lola_decode_step scores the cached pairs (same result, other cost):
 *   LOLA_DECODE_RESCORE      every step computes H^T phi(k) and s . phi(k) for
 *                            every cached pair against the step-start state (the
 *                            summary's "Inferentiestrategie", step 1, as written)
 *   LOLA_DECODE_INCREMENTAL  the state keeps, per cached pair, n = H^T phi(k) and
 *                            d = s . phi(k); a step scores the cache from them and
 *                            adds the one folded pair's share, (phi(k) . phi(k_f))
 *                            times [v_f; 1], instead of recomputing them: O(C (F + D))
 *                            work per step instead of O(C F D), against 4 (D + 1)
 *                            more bytes of state per cached pair read and written.
 *                            bf16 io and LOLA_POLICY_SRE only.  A prefill call
 *                            marks the stored n, d stale; the next decode step
 *                            recomputes them in full. */
typedef enum { LOLA_DECODE_RESCORE = 0, LOLA_DECODE_INCREMENTAL = 1 } lola_decode_mode;

typedef enum {
    LOLA_POLICY_SRE = 0,
    LOLA_POLICY_SRE_STALE = 1,
    LOLA_POLICY_FIFO = 2,
    LOLA_POLICY_ATTN = 3,
    LOLA_POLICY_SOFTMAX_ERR = 4
} lola_policy;

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
    int32_t policy;        /* one of lola_policy; 0 = the SRE of the method */
    int32_t decode_mode;   /* one of lola_decode_mode; 0 = rescore every cached pair */
} lola_config;

/* Bytes of the state buffer for `batch` sequences: a header, W, and per
 * (sequence, KV head) the three memories of the summary's "Methodologie:
 * LoLA" section -- the sliding window (ring of the last `window` keys and
 * values), the sparse cache (positions, keys, values, and for bf16 io the
 * feature-map pre-activations z = W k of the cached keys) and the recurrent
 * state H [F][D] f32,
 * s [F] f32 -- plus the tokens seen.  The size does not grow with the
 * sequence length.  0 if the config or batch is not supported. */
size_t lola_state_bytes(const lola_config* cfg, int32_t batch);

/* Bytes of scratch that lola_prefill_chunk needs for up to `max_tokens`
 * tokens per call (feature rows, interval-start snapshots of H, s and the
 * cache, copies of the window and cache at the call start).  0 if invalid. */
size_t lola_prefill_workspace_bytes(const lola_config* cfg, int32_t batch, int32_t max_tokens);

/* Initialise `state` (device, lola_state_bytes) for `batch` empty sequences:
 * header, tokens seen = 0, H = 0, s = 0, empty cache and window -- the three
 * memories of "Methodologie: LoLA" before any pair has been seen.
 * W: device [n_kv_heads][feat_half][head_dim] f32, copied into the state; it
 * defines the feature map phi(x) = [softmax(W x); softmax(-W x)] (the paper
 * abstract only calls it a low-rank feature map; this form is the
 * library's).  Errors: LOLA_ERR_INVALID_ARG for a NULL or misaligned W or
 * state, LOLA_ERR_UNSUPPORTED for a config outside the supported set. */
lola_status lola_init_state(const lola_config* cfg, int32_t batch, const float* W, void* state,
                            void* stream);

/* Advance every sequence by n_tokens (> 0) tokens in the chunkwise mode of
 * the summary's "Inferentiestrategie" section: positions
 * [t0, t0 + n_tokens) are processed as consecutive update intervals of
 * cfg->chunk tokens (the last may be shorter), each call starting its own
 * interval grid at t0.  Per interval: outputs of its queries from the
 * interval-start memories (step 4), then SRE scoring of leaving + cached
 * pairs (step 1), top-C keep (step 2), fold of the rest (step 3), window
 * update.
 * Errors (host side, before any launch): LOLA_ERR_INVALID_ARG for NULL or
 * misaligned pointers or n_tokens < 1, LOLA_ERR_UNSUPPORTED for a config or
 * batch outside the supported set, LOLA_ERR_WORKSPACE for a short workspace,
 * LOLA_ERR_HIP for a failed launch; device side, see the state header above.
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

/* lola_prefill_chunk for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid hipMalloc): the same
 * computation and results, with the workspace taken from a library-owned
 * static device array of LOLA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, which
 * each GPU the library runs on holds from its first use until the process
 * ends.  This call allocates and frees nothing (the first call on a device
 * only looks up that device's copy of the array).
 *   Errors: as lola_prefill_chunk, and LOLA_ERR_WORKSPACE if
 *   lola_prefill_workspace_bytes(cfg, batch, n_tokens) exceeds
 *   LOLA_NOALLOC_SCRATCH_BYTES (e.g. more than one 4096-token call of the
 *   32/8-head, head_dim 128 layer at batch 1), LOLA_ERR_INVALID_ARG if
 *   `stream` belongs to a device other than the current one.
 *   Every call on one GPU shares the array: calls that overlap in time on one
 *   GPU (other streams, other host threads) race and must be serialised by
 *   the caller; calls in order on one stream are safe. */
#define LOLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lola_status lola_prefill_chunk_noalloc(const lola_config* cfg, void* state, int32_t batch, int32_t n_tokens,
                                       const void* q, const void* k, const void* v, void* out, void* stream);

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

/* One token for every sequence: the token-by-token mode of the summary's
 * "Inferentiestrategie" section (its steps 1-4 on a one-token interval), in
 * one fused launch that needs no workspace.  It computes what
 * lola_prefill_chunk(n_tokens = 1) computes and keeps the same pair (SRE
 * descending, position ascending); the arithmetic differs (the fold of the
 * one evicted pair runs in fp32 vector FMAs instead of MFMAs, the softmax in
 * other blocks), so outputs and H, s agree within the io dtype's tolerance
 * rather than bit for bit.
 *   q [batch][n_q_heads][head_dim], k, v [batch][n_kv_heads][head_dim],
 *   out [batch][n_q_heads][head_dim], all io dtype.
 * Errors: as lola_prefill_chunk (no workspace). */
lola_status lola_decode_step(const lola_config* cfg, void* state, int32_t batch, const void* q,
                             const void* k, const void* v, void* out, void* stream);

/* Copy the memories out of `state` into caller device buffers (any output
 * may be NULL): the sparse cache and the recurrent state H, s of
 * "Methodologie: LoLA", e.g. to inspect which pairs the SRE kept
 * ("Inferentiestrategie", step 2).  Cache entries are written in ascending
 * position order.  A state whose header does not match the config and batch
 * leaves every output unwritten (a faulted state is still read).
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
