/*
 * sparsekv.h -- C ABI of the MI355X (gfx950) sparse-KV decode step.
 *
 * One decode step of one attention layer, for a batch of sequences, in three
 * stages (page "8 agents x 250K context on two 3090s: sparse KV decode with a
 * rank-64 key sketch and a host-RAM tier", section "The mechanism"; page
 * "3.14M Context on 3x 3090: The Power of an Architecture That Puts KV Cache
 * in Host RAM", sections "Why" and "What Needs to Stay in VRAM"):
 *
 *   score   a cheap indexer scores every past token through a rank-64 int4
 *           key sketch (token mode) or every complete 4-token block through
 *           a mean-pooled 128-dim bf16 indexer key (block mode);
 *   select  a deterministic top-k keeps the best `topk` tokens (or blocks),
 *           one pick per layer shared by all KV heads, joined with the sink
 *           tokens and the recent tail (token mode) or the trailing partial
 *           block (block mode); short sequences are attended densely;
 *   attend  exact GQA softmax attention over only the selected K/V rows.
 *
 * plus an optional host-RAM KV tier: K/V stored at int4 in pinned host
 * memory, read zero-copy by the GPU for the picked rows that miss a GPU hot
 * buffer (2.5% of tokens, windowed CLOCK), turned back into int8 rows on fetch.
 *
 * Conventions shared by every call:
 *  - All array arguments are DEVICE pointers unless stated otherwise, owned by
 *    the caller, and must stay valid until the enqueued work has finished.
 *    The library keeps no pointer after a step call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Step
 *    calls (qsketch, score, topk, attend, step, tier_resolve) only enqueue
 *    kernels on that stream: they never synchronize, never allocate and never
 *    record a memset, so they can be captured into a HIP graph.
 *  - Errors found on the host (bad descriptor, NULL pointer, workspace too
 *    small) return a status and enqueue nothing; sparsekv_last_error() gives
 *    a thread-local message.  A failed kernel launch returns SKV_ERR_HIP.
 *    Conditions only visible on the device (a ctx_len outside [0, max_ctx],
 *    an index outside its array) are clamped or skipped by the kernels and
 *    recorded as flag bits in the workspace; sparsekv_check() reads them.
 *  - Calls are reentrant with distinct workspaces.  Two calls that share a
 *    workspace, or a tier handle, must be ordered on one stream.
 */
#ifndef SPARSEKV_H
#define SPARSEKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSEKV_ABI_VERSION 7   /* 3: multi-query step, prefill over host K/V, tier policy field;
                                    4: tier append (host records sized by max_ctx, tail ring),
                                       multi-query tier resolve and attention;
                                    5: the step without a workspace argument;
                                    6: tier page residency (desc fields, map / unmap, in_place
                                       counter), tier_attend, tier_host_ptr;
                                    7: contraction path switch (measurement aid) */

typedef int32_t skv_status;
enum {
  SKV_OK = 0,
  SKV_ERR_INVALID = 1,      /* bad argument or descriptor */
  SKV_ERR_UNSUPPORTED = 2,  /* valid but not implemented (shape/dtype) */
  SKV_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than sparsekv_workspace_size */
  SKV_ERR_OOM = 4,          /* device or host allocation failed (tier_create only) */
  SKV_ERR_HIP = 5,          /* a HIP runtime call or kernel launch failed */
  SKV_ERR_HOST_MEMORY = 6,  /* host records not pinned/mappable for device access */
  SKV_ERR_STATE = 7,        /* device flags were raised (see sparsekv_check) */
};

/* index (scoring) modes */
enum { SKV_INDEX_SKETCH_INT4 = 0, SKV_INDEX_POOLED_BF16 = 1 };
/* K/V storage formats */
enum { SKV_KV_I8_ROWSCALE = 0, SKV_KV_F16 = 1, SKV_KV_BF16 = 2 };
/* query formats */
enum { SKV_Q_F16 = 0, SKV_Q_BF16 = 1 };

/* device flag bits reported by sparsekv_check */
enum {
  SKV_FLAG_CTX_RANGE = 1u << 0,    /* a ctx_len was < 0 or > max_ctx (clamped) */
  SKV_FLAG_INDEX_RANGE = 1u << 1,  /* attend: an index outside [0, rows) or n_sel > cap (skipped/clamped) */
  SKV_FLAG_TOPK_SLOW = 1u << 2,    /* informational: a sequence needed the exact slow select path */
  SKV_FLAG_TIER_INPUT = 1u << 3,   /* tier: a pick outside [0, ctx) or unsorted input (skipped) */
  SKV_FLAG_WAIT = 1u << 4,         /* a workgroup stopped waiting for another of its sequence (results incomplete) */
};

/*
 * Layer descriptor (plain old data).
 *
 * Token mode (index_mode = SKV_INDEX_SKETCH_INT4): block = 1, rank = 64 (a
 * multiple of 16 in [16, 256] with n_kv_heads*rank/2 in {32, 64, 128, 256}),
 * topk = tokens kept from the middle range [n_sink, T - n_tail); a sequence
 * is dense (all T tokens attended) when T <= n_sink + topk + n_tail.
 *
 * Block mode (index_mode = SKV_INDEX_POOLED_BF16): block = 4, index_dim = 128
 * (any multiple of 8), topk = blocks kept; n_sink = n_tail = 0.  Only the
 * floor(T/4) complete blocks are scored; the T mod 4 trailing tokens are
 * always attended; dense when floor(T/4) <= topk, i.e. T <= 4*topk + 3.
 *
 * T = ctx_len[b] counts the tokens in the cache including the current one.
 * Supported: head_dim in {128, 256}, n_q_heads / n_kv_heads in [1, 16],
 * K/V int8 + fp16 row scale (head_dim 256) or fp16 (token mode), bf16 (block
 * mode), topk <= 4096, at most 16384 selected positions per sequence.
 */
typedef struct {
  uint32_t struct_size;   /* sizeof(skv_layer_desc) */
  int32_t batch;          /* sequences B */
  int32_t max_ctx;        /* per-sequence capacity (row stride) of every [B][max_ctx]... array */
  int32_t n_kv_heads;     /* H_kv */
  int32_t n_q_heads;      /* H_q (multiple of H_kv) */
  int32_t head_dim;       /* D */
  int32_t index_mode;     /* SKV_INDEX_* */
  int32_t rank;           /* R: sketch rank per KV head (token mode) */
  int32_t index_dim;      /* pooled indexer key width (block mode) */
  int32_t block;          /* 1 (token mode) or 4 (block mode) */
  int32_t topk;           /* budget: tokens (token mode) or blocks (block mode) */
  int32_t n_sink;         /* S */
  int32_t n_tail;         /* L */
  int32_t kv_dtype;       /* SKV_KV_* */
  int32_t q_dtype;        /* SKV_Q_* */
} skv_layer_desc;

/* A view of K/V rows: element (b, row, h, d) of K is at
 *   k + ((b * rows + row) * n_kv_heads + h) * head_dim + d
 * (page "3.14M Context on 3x 3090 ...", section "No Need to Rewrite the
 * Kernel": rows are addressed by (token * n_kv_heads + kv_head) * head_dim).
 * Row scales (SKV_KV_I8_ROWSCALE only) are fp16 at (b * rows + row) * n_kv_heads + h. */
typedef struct {
  const void* k;
  const void* v;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  int64_t rows;           /* rows per sequence (max_ctx for the plain cache) */
} skv_kv_view;

/* ---- library ------------------------------------------------------------ */

int sparsekv_abi_version(void);
const char* sparsekv_status_str(skv_status s);
/* Thread-local detail of the last error returned on this thread ("" if none). */
const char* sparsekv_last_error(void);

/* Validates a descriptor on the host.  SKV_OK, SKV_ERR_INVALID or SKV_ERR_UNSUPPORTED. */
skv_status sparsekv_validate(const skv_layer_desc* d);

/* Largest number of positions select can emit per sequence:
 * n_sink + topk + n_tail (token mode) or 4*topk + 3 (block mode). */
skv_status sparsekv_select_capacity(const skv_layer_desc* d, int32_t* cap);

/* Device workspace bytes the step calls need for this descriptor.  The caller
 * allocates it once, 256-byte aligned, zero-fills it once (its first word is
 * the device flag word that sparsekv_check reads and clears; every other byte
 * is initialised by the calls that use it) and passes it to every step call. */
skv_status sparsekv_workspace_size(const skv_layer_desc* d, size_t* bytes);

/* ---- stage A1: query sketch (token mode) ----------------------------------
 * Page "8 agents x 250K ...", section "The mechanism": every token is scored
 * through a rank-R projection onto a frozen basis, one pick per layer shared
 * by the KV heads; the query side is an int8 vector.
 *   q        [B][H_q][D] fp16
 *   basis    [H_kv][D][R] fp32 (basis vector r of KV head h is basis[h][:][r])
 *   qs       [B][H_kv*R] int8 out:  clamp(rint(s/qscale), +-127) where, per KV
 *            head h, s_h = sum over d ascending of (qbar_h[d] * basis_h[d][r])
 *            with qbar_h = sum of the G query heads of h in ascending order,
 *            all in fp32 with separately rounded multiplies and adds;
 *   qs_scale [B] fp32 out: max|s| / 127 (0 when the sketch is all zero).
 * Uses the workspace (the fp32 sketch before quantization). */
skv_status sparsekv_qsketch(const skv_layer_desc* d, const void* q, const float* basis,
                            int8_t* qs, float* qs_scale, void* ws, size_t ws_bytes, void* stream);

/* ---- stage A2: exact ranking keys -----------------------------------------
 * Token mode (page "8 agents x 250K ...", section "The mechanism"):
 *   index_query = qs [B][H_kv*R] int8; index_keys = int4 codes
 *   [B][max_ctx][H_kv*R/2] uint8 (element 2j in the low nibble of byte j,
 *   two's complement); index_scale = per-token fp16 scale [B][max_ctx];
 *   keys[b][t] = (double)(sum_i qs[i]*code_t[i]) * (double)scale_t  (exact)
 *   for every middle token t in [n_sink, T - n_tail); keys is [B][max_ctx].
 * Block mode (page "3.14M Context ...", sections "Why", "What Needs to Stay in
 * VRAM"): index_query = [B][index_dim] bf16; index_keys = pooled keys
 *   [B][max_ctx/4][index_dim] bf16; index_scale = NULL;
 *   keys[b][j] = sum_i q[i]*kp_j[i] accumulated in fp64 for every complete
 *   block j < floor(T/4); keys is [B][max_ctx/4].  The sum is exact (hence
 *   identical to any other evaluation order) when every bf16 input is 0 or of
 *   magnitude in [2^-8, 2^8).
 * Other entries of keys are not written.  -0 is written as +0. */
skv_status sparsekv_score(const skv_layer_desc* d, const int32_t* ctx_len,
                          const void* index_query, const void* index_keys,
                          const uint16_t* index_scale, double* keys,
                          void* ws, size_t ws_bytes, void* stream);

/* ---- stage A3: deterministic top-k + sinks/tail ---------------------------
 * Pages: "8 agents x 250K ...", section "The mechanism" (deterministic top-k,
 * sinks, tail, dense/sparse switch); "3.14M Context ...", section "Why" (dense
 * until the context exceeds 4*block_topk+3, then exactly the budget).
 * Keeps the `topk` candidates with the largest keys, equal keys going to the
 * lower position, and writes for each sequence the ascending unique token
 * positions to attend:
 *   token mode: [0, S) + top-k of [S, T-L) + [T-L, T), or [0, T) when dense;
 *   block mode: the 4 tokens of each kept block + [4*floor(T/4), T), or [0, T).
 *   idx   [B][cap] int32 out (cap from sparsekv_select_capacity; entries past
 *         n_sel[b] are unspecified); n_sel [B] int32 out. */
skv_status sparsekv_topk(const skv_layer_desc* d, const int32_t* ctx_len, const double* keys,
                         int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream);

/* Stages A2 + A3 in one call, without materializing the keys: idx / n_sel
 * are identical to sparsekv_topk applied to the keys sparsekv_score would
 * write.  The index is streamed once; the keys at or above a threshold
 * estimated from a sample of the index are kept in the workspace as
 * (key, position) candidates and the exact select runs on them (on every key,
 * recomputed, in the rare case the candidates are fewer than topk; that case
 * raises SKV_FLAG_TOPK_SLOW). */
skv_status sparsekv_score_topk(const skv_layer_desc* d, const int32_t* ctx_len,
                               const void* index_query, const void* index_keys,
                               const uint16_t* index_scale, int32_t* idx, int32_t* n_sel,
                               void* ws, size_t ws_bytes, void* stream);

/* ---- stage A4: exact GQA attention over the selected rows -----------------
 * Page "8 agents x 250K ...", section "The mechanism" (exact attention on the
 * kept tokens); page "3.14M Context ...", section "No Need to Rewrite the
 * Kernel" (gather by row offset).
 *   q    [B][H_q][D] fp16 (bf16 for bf16 K/V)
 *   kv   rows to gather from; idx [B][cap] row indices, n_sel [B] counts
 *   out  [B][H_q][D] fp32: for query head j of KV head h = j / (H_q/H_kv),
 *        softmax over the n_sel rows of (q_j . k_row) * sm_scale, times V;
 *        K/V int8 rows are code * fp16 row scale.  n_sel = 0 gives zeros. */
skv_status sparsekv_attend(const skv_layer_desc* d, const void* q, const skv_kv_view* kv,
                           const int32_t* idx, const int32_t* n_sel, float sm_scale, float* out,
                           void* ws, size_t ws_bytes, void* stream);

/* ---- the whole step --------------------------------------------------------
 * A1..A4 in one call: sparsekv_qsketch (token mode), sparsekv_score_topk and
 * sparsekv_attend.  Token mode: basis, qs, qs_scale are used and qs / qs_scale
 * written; block mode: they may be NULL and index_query is the bf16 indexer
 * query.  qs, qs_scale, idx, n_sel, out are written as by the separate calls. */
skv_status sparsekv_step(const skv_layer_desc* d, const int32_t* ctx_len, const void* q,
                         const float* basis, int8_t* qs, float* qs_scale,
                         const void* index_query, const void* index_keys,
                         const uint16_t* index_scale, const skv_kv_view* kv, int32_t* idx,
                         int32_t* n_sel, float sm_scale, float* out, void* ws, size_t ws_bytes,
                         void* stream);

/* ---- the whole step without a workspace argument ----------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Computes
 * exactly what sparsekv_step computes, with the same arguments except
 * ws / ws_bytes, in a device array of SKV_NOALLOC_SCRATCH_BYTES inside the
 * library (one per device, kept until the process ends) instead of a caller
 * workspace; nothing is allocated.
 *   flags   device uint32 (may be NULL): receives this call's device flag
 *           word (the bits sparsekv_check reports for sparsekv_step); the
 *           library's copy is cleared at the end of every call
 *   errors  SKV_ERR_WORKSPACE when the layer needs more scratch than the array
 *           holds (sparsekv_workspace_size(d) > SKV_NOALLOC_SCRATCH_BYTES: in
 *           token mode batch x max_ctx above about 4M tokens); otherwise as
 *           sparsekv_step
 * Runs on the device current at the call (the stream must belong to it).
 * Every call on one device uses the same array: calls ordered on one stream
 * are safe, calls that overlap in time on one device (other streams, other
 * host threads) race and give wrong results. */
#define SKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
skv_status sparsekv_step_noalloc(const skv_layer_desc* d, const int32_t* ctx_len, const void* q,
                                 const float* basis, int8_t* qs, float* qs_scale,
                                 const void* index_query, const void* index_keys,
                                 const uint16_t* index_scale, const skv_kv_view* kv, int32_t* idx,
                                 int32_t* n_sel, float sm_scale, float* out, uint32_t* flags,
                                 void* stream);

/* ---- the step with several query tokens per sequence ------------------------
 * Page "8 agents x 250K ...", section "What shipped" (decoding with MTP-7
 * speculation: one step verifies the drafted tokens with the current one) and
 * section "The mechanism"; page "vLLM's Hybrid HiSparse Triples Concurrent
 * Requests on Million-Token Contexts", section "Where the tradeoffs bite"
 * (every verification token has its own pick).  Token mode only, with
 * H_kv*R/2 in {64, 128, 256} sketch bytes per token.
 *   n_query  M in [1, 16]: the query tokens of each sequence are the last M
 *            positions of its cache (ctx_len[b] = T counts them); query j
 *            sees the causal context T_j = T - M + 1 + j (0 if negative) and
 *            gets exactly what sparsekv_step computes for a single query at
 *            ctx_len T_j: its own int8 sketch and scale, its own top-k over
 *            [n_sink, T_j - n_tail), sinks and tail of T_j, dense when
 *            T_j <= n_sink + topk + n_tail, and exact attention (T_j = 0:
 *            nothing selected, zero output)
 *   q        [B][M][H_q][D] fp16
 *   qs       [B][M][H_kv*R] int8 (16-byte aligned), qs_scale [B][M] fp32: written
 *   idx      [B][M][cap], n_sel [B][M], out [B][M][H_q][D] fp32: written
 *   ws       sparsekv_workspace_size_multi(d, M) bytes, 256-byte aligned
 * The sketch is read once per step for all M queries (an int8 matrix-core
 * contraction of the codes with the M query sketches).  Other arguments and
 * errors as sparsekv_step. */
skv_status sparsekv_workspace_size_multi(const skv_layer_desc* d, int32_t n_query, size_t* bytes);
skv_status sparsekv_step_multi(const skv_layer_desc* d, int32_t n_query, const int32_t* ctx_len,
                               const void* q, const float* basis, int8_t* qs, float* qs_scale,
                               const void* index_keys, const uint16_t* index_scale,
                               const skv_kv_view* kv, int32_t* idx, int32_t* n_sel, float sm_scale,
                               float* out, void* ws, size_t ws_bytes, void* stream);
/* The attention of sparsekv_step_multi alone: query token j of sequence b
 * (q [B][n_query][H_q][D], same dtype rules as sparsekv_attend) attends the
 * rows idx[b][j][0..n_sel[b][j]) of sequence b's K/V view; out fp32
 * [B][n_query][H_q][D].  Workspace: sparsekv_workspace_size_multi. */
skv_status sparsekv_attend_multi(const skv_layer_desc* d, int32_t n_query, const void* q,
                                 const skv_kv_view* kv, const int32_t* idx, const int32_t* n_sel,
                                 float sm_scale, float* out, void* ws, size_t ws_bytes,
                                 void* stream);

/* ---- prefill attention over K/V rows in host memory -------------------------
 * Page "3.14M Context ...", sections "What Needs to Stay in VRAM" (K and V in
 * host RAM) and "The Downside to Keep in Mind": every prefill token has its
 * own pick, so the history is streamed once in fixed-size chunks through a
 * small device buffer, all queries are computed against each chunk and their
 * partial softmax results merged.  The bytes copied are the history once,
 * whatever chunk_bytes is.
 *   d          layer shape: n_kv_heads, n_q_heads, head_dim; kv_dtype SKV_KV_F16
 *              or SKV_KV_BF16 with the matching q_dtype
 *   n_query    P >= 1 query tokens
 *   q          device [P][H_q][D] fp16 / bf16
 *   idx        device [P][cap] int32: query p's picked positions, ascending and
 *              < n_tokens, in its first n_sel[p] entries (n_sel device [P])
 *   host_k, host_v  host [n_tokens][H_kv][D] rows (fp16 / bf16); pinned memory
 *              (hipHostMalloc) is copied by DMA, pageable memory is staged by
 *              the runtime
 *   chunk_buf  device working buffer of chunk_bytes, 16-byte aligned, used as two
 *              halves: chunks of floor(chunk_bytes / (4*H_kv*D*2)) tokens' K and
 *              V rows, one half filled while the other is read
 *   out        device [P][H_q][D] fp32: softmax of (q_j . k_t)*sm_scale over
 *              query p's listed rows t, times V (KV head of query head j is
 *              j / (H_q/H_kv)); zeros when n_sel[p] = 0
 *   ws         sparsekv_prefill_workspace_size(d, P) bytes, 256-byte aligned: a
 *              flag word (read by sparsekv_check), then the running (max, sum)
 *              and accumulator of every query head
 * Enqueues on `stream` a state reset, per chunk one kernel and the
 * normalisation; the host-to-device copies run on a copy stream the library
 * keeps per device, ordered against `stream` by events (a copy starts after
 * the work already on `stream`; every kernel waits for its chunk's copy; a
 * half is refilled after the kernel that read it).  Returns without waiting;
 * once `stream` has passed the call, all of its work is done.  The host rows
 * and all buffers must stay valid until then.  Calls from several host
 * threads on one device are serialised while they enqueue.  An
 * index outside [0, n_tokens) or n_sel outside [0, cap] is skipped / clamped
 * and raises SKV_FLAG_INDEX_RANGE; so does a list entry found outside the
 * chunk being processed (an unsorted list). */
skv_status sparsekv_prefill_workspace_size(const skv_layer_desc* d, int32_t n_query, size_t* bytes);
skv_status sparsekv_prefill_attend(const skv_layer_desc* d, int32_t n_query, const void* q,
                                   const int32_t* idx, const int32_t* n_sel, int32_t cap,
                                   const void* host_k, const void* host_v, int64_t n_tokens,
                                   void* chunk_buf, size_t chunk_bytes, float sm_scale, float* out,
                                   void* ws, size_t ws_bytes, void* stream);

/* ---- append: the new token of every sequence into the caches ---------------
 * Page "8 agents x 250K ...", section "The mechanism" (int8 K/V rows with a
 * per-row scale, int4 rank-64 key sketch with one fp16 scale per token); page
 * "3.14M Context ...", section "No Need to Rewrite the Kernel" (the paged cache
 * update writes the new rows in place each step).  Token mode only.
 *   ctx_len     [B] int32, read and written: the token goes to row ctx_len[b]
 *               of sequence b, then ctx_len[b] += 1; a sequence already at
 *               max_ctx is left unchanged and raises SKV_FLAG_CTX_RANGE
 *   k_new,v_new [B][H_kv][D] fp16: the new token's key and value rows
 *   basis       [H_kv][D][R] fp32, the frozen sketch basis
 *   kv          the cache (rows >= max_ctx): int8 rows + fp16 row scales,
 *               scale = fp16(fp32(amax/127)), code = clamp(rint(x/scale), +-127)
 *               (zero row -> scale 0); fp16 K/V caches get the rows as they are
 *   index_keys  [B][max_ctx][H_kv*R/2] u8, index_scale [B][max_ctx] fp16: the
 *               sketch v[h*R+r] = sum over d ascending of k_h[d]*B_h[d][r]
 *               (fp32, no fused multiply-add), scale fp16(fp32(amax/7)) over
 *               all H_kv*R values, codes clamp(rint(v/scale), +-7), element 2j
 *               in the low nibble of byte j
 * Quotients are correctly rounded fp32.  Uses the workspace's flag word only. */
skv_status sparsekv_append(const skv_layer_desc* d, int32_t* ctx_len, const void* k_new,
                           const void* v_new, const float* basis, const skv_kv_view* kv,
                           void* index_keys, uint16_t* index_scale, void* ws, size_t ws_bytes,
                           void* stream);

/* Block mode (page "3.14M Context ...", sections "Why" and "What Needs to
 * Stay in VRAM": a 4-token block's indexer key is the mean of its tokens' raw
 * indexer keys, bf16).
 *   ctx_len      [B] int32, read and written as in sparsekv_append
 *   k_new,v_new  [B][H_kv][D] bf16, stored as they are in the bf16 cache kv
 *   index_raw    [B][index_dim] bf16: the new token's raw indexer key
 *   index_stage  [B][4][index_dim] bf16, caller-owned and kept per layer
 *                across steps: row t % 4 receives the raw key of token t
 *                (after a prefill that ends inside a block it must hold that
 *                block's raw keys)
 *   index_keys   [B][max_ctx/4][index_dim] bf16: when t % 4 == 3 the pooled
 *                key of block t/4 = the exact mean of the four staged keys,
 *                rounded to nearest-even bf16, 0 below 2^-8 in magnitude,
 *                clamped to +-255 (the domain in which scores are exact) */
skv_status sparsekv_append_block(const skv_layer_desc* d, int32_t* ctx_len, const void* k_new,
                                 const void* v_new, const void* index_raw, void* index_stage,
                                 const skv_kv_view* kv, void* index_keys, void* ws,
                                 size_t ws_bytes, void* stream);

/* Synchronizes `stream`, returns the device flag bits raised since the last
 * check in *flags (may be NULL) and clears them.  SKV_ERR_STATE if any bit
 * other than SKV_FLAG_TOPK_SLOW was set.  Not capturable. */
skv_status sparsekv_check(void* ws, size_t ws_bytes, void* stream, uint32_t* flags);

/* ---- diagnostic kernel timer -------------------------------------------------
 * For measurement only (not thread-safe, not capturable).  While enabled, every
 * launch of one kind of kernel carries a start/stop event pair that its
 * dispatch records (hipExtLaunchKernelGGL), so the pair spans the kernel's
 * execution.  enable = 0 turns the timer off; SKV_TIMER_ATTEND times the
 * attention kernel (sparsekv_attend, sparsekv_step, sparsekv_step_multi; not
 * the merge of its partials); any other nonzero value (SKV_TIMER_STREAM) times
 * the dominant kernel of a call: the streaming score-and-collect kernel (the
 * one that reads the whole index in sparsekv_score_topk, sparsekv_step,
 * sparsekv_step_multi), the resolver of sparsekv_tier_resolve (it fetches the misses) and the
 * kernel of sparsekv_append and sparsekv_tier_append.  Up to 4096 launches are recorded.  Enabling again
 * discards earlier records.  sparsekv_timer_read synchronizes on the recorded
 * events and returns the summed kernel time (ms) and the number of launches. */
#define SKV_TIMER_STREAM 1
#define SKV_TIMER_ATTEND 2
skv_status sparsekv_timer_enable(int enable);
skv_status sparsekv_timer_read(double* total_ms, int64_t* launches);
/* ---- measurement aid: a plain streaming read ---------------------------------
 * Not a step of the method: the reference rate for its dominant read.  Page
 * "3.14M Context on 3x 3090 ...", section "What Needs to Stay in VRAM" (the
 * index scan is the per-step read that grows with context) and page "8 agents
 * x 250K ...", section "The mechanism" (misses read host memory over PCIe):
 * reading the same bytes with no arithmetic bounds what the scan (device
 * memory) or the zero-copy fetch (mapped host memory) can reach.
 *   src    device address of device memory or of mapped pinned host memory,
 *          16-byte aligned; every 16-byte word of [src, src + bytes) is loaded
 *          once (bytes a multiple of 16)
 *   sink   device uint32 [n_wg]: each workgroup stores the xor of its words
 *   n_wg   workgroups of 256 threads, 1 .. SKV_READ_MAX_WG
 * Timed by sparsekv_timer_enable(SKV_TIMER_STREAM) like the dominant kernels. */
#define SKV_READ_MAX_WG 65536
skv_status sparsekv_read_bytes(const void* src, size_t bytes, uint32_t* sink, int32_t n_wg,
                               void* stream);

/* ---- measurement aid: the dense contractions on the vector ALUs -------------
 * Not a step of the method: selects the units that compute the path's two
 * dense contractions, to measure what the matrix cores bring.
 *   SKV_PATH_MFMA (the default): matrix-core tiles.
 *   SKV_PATH_VALU: kernels with the same grid, data layout and outputs that
 *     compute on the vector ALUs.
 * The contractions:
 *   - single-query attention over int8 K/V with row scales (one query per
 *     sequence, head_dim 128 or 256, at most 7 query heads per KV head at
 *     head_dim 256 or 12 at 128, the 8-wave workgroup shape) in
 *     sparsekv_attend, sparsekv_step, sparsekv_step_noalloc and
 *     sparsekv_tier_attend; page "8 agents x 250K ...", section "The
 *     mechanism" (exact attention over the gathered rows).  Matrix cores: fp16
 *     tiles, the probabilities entering P.V as two fp16 parts; vector ALUs:
 *     fp32 dot products.  Outputs agree to fp32 rounding.
 *   - the multi-query sketch score (sparsekv_step_multi, sketch rows of at
 *     most 128 bytes); same page, section "What shipped" (the drafted tokens
 *     verified in one step).  Matrix cores: int8 tiles; vector ALUs: 4-way
 *     int8 dot instructions.  Integer arithmetic: index sets and keys are
 *     bit-identical.
 * Every other shape takes the matrix-core kernel.  Process-wide and not
 * thread-safe: set it between calls.  SKV_ERR_INVALID for any other value. */
#define SKV_PATH_MFMA 0
#define SKV_PATH_VALU 1
skv_status sparsekv_set_contraction_path(int32_t path);

/* ---- host-RAM tier (optional) ----------------------------------------------
 * Page "8 agents x 250K ...", section "The mechanism": K/V of every token sit
 * in pinned host RAM at int4 (64-dim groups, fp16 group scales, 272 B per
 * token-head at head_dim 256); the GPU keeps the sketch, the sinks, the tail
 * and a hot buffer of 2.5% of the tokens under windowed CLOCK; misses read only
 * the picked rows over PCIe and are turned back into int8 rows.  Page "3.14M
 * Context ...", section "No Need to Rewrite the Kernel": zero-copy access to
 * mapped host memory needs no per-layer host synchronization.
 *
 * Host record of token t, KV head h (record bytes = 2 * (D/2 + 2*D/64)):
 *   K: D/2 bytes of int4 codes (low nibble first) then D/64 fp16 group scales,
 *   V: the same; records are [B][max_ctx][H_kv][record] token-major (the
 *   layer's max_ctx is the tier's capacity; the caller fills positions
 *   [0, ctx), sparsekv_tier_append writes the later ones).
 * Fetch turns a row into int8 with one fp16 scale s' = fp16(gmax*7/127),
 * gmax the largest group scale, and r8 = clamp(rint(c*g / s'), +-127), each
 * operation one fp32 IEEE operation (c*g and gmax*7 are exact).
 *
 * Resident rows per sequence (an skv_kv_view, int8 + fp16 row scales):
 *   [0, S) sinks, [S, S+L) tail, [S+L, S+L+n_slots) hot slots,
 *   [S+L+n_slots, S+L+n_slots + pool_pages*page_tokens) the page pool.  The tail is a
 *   ring anchored at the creation context ctx0 = desc.ctx: tail position p
 *   sits in row S + ((p - ctx0) mod L), so at creation row S+i holds position
 *   ctx0-L+i.  The caller loads sinks and tail once, before any append, with
 *   sparsekv_tier_load_resident.  Each sequence's context T starts at ctx0 and
 *   is kept on the device; sparsekv_tier_append advances it.
 *
 * Windowed CLOCK, per sequence and step s: picked tokens already in the hot
 * buffer are hits (ref=1, last=s); the misses, in ascending position order,
 * each take the first slot the hand reaches that is empty, or unused for the
 * last W steps (last <= s-W) and unreferenced -- a referenced slot outside
 * the window has its reference cleared as the hand passes it.
 *
 * Page residency (page "vLLM's Hybrid HiSparse Triples Concurrent Requests on
 * Million-Token Contexts", section "Three residency states, one block pool"):
 * with page_tokens P > 0 the positions of a sequence form pages of P
 * (page = p / P) and each page is either mapped to a block of the sequence's
 * device pool -- its int8 rows resident, read in place -- or a placeholder
 * whose picks go through the hot buffer from host memory.  Every page mapped
 * is full residency, some mapped is mixed residency, none is no residency
 * (the default); sinks and tail are resident in every state.  The caller
 * decides, between steps, which pages to map (sparsekv_tier_map_page copies
 * a page's rows into a block) and which to give up (sparsekv_tier_unmap_page),
 * e.g. under memory pressure; a middle pick of a mapped page p sits in
 * resident row S+L+n_slots + block*P + p%P and counts as in_place. */
typedef struct skv_tier skv_tier;

/* Hot-buffer policies.  SKV_TIER_CLOCK: the windowed CLOCK above.
 * SKV_TIER_LRU -- page "vLLM's Hybrid HiSparse Triples Concurrent Requests on
 * Million-Token Contexts", section "Three residency states, one block pool"
 * (a hot row's LRU entry is refreshed on use, a miss copies its row into an
 * LRU slot; hot buffers of 2x top-K rows by default): hits set the slot's last
 * use to the step; the misses take the slots not used in this step, oldest
 * last use first (an empty slot before any used one, equal last uses in slot
 * order), and fill them in ascending slot order in ascending position order.
 * window is ignored; n_slots >= topk. */
enum { SKV_TIER_CLOCK = 0, SKV_TIER_LRU = 1 };

typedef struct {
  uint32_t struct_size;   /* sizeof(skv_tier_desc) */
  skv_layer_desc layer;   /* token mode, SKV_KV_I8_ROWSCALE */
  int32_t ctx;            /* tokens per sequence at creation (ctx0 <= layer.max_ctx) */
  int32_t n_slots;        /* hot slots per sequence; must exceed topk */
  int32_t window;         /* W >= 1 */
  void* host_records;     /* NULL: the library allocates pinned, device-mapped
                             host memory; otherwise caller memory that is
                             already pinned and mapped (e.g. hipHostMalloc) */
  int32_t policy;         /* SKV_TIER_*; a struct_size that ends before this
                             field means SKV_TIER_CLOCK */
  int32_t page_tokens;    /* P: 0 (no page table) or a power of two in [16, 4096];
                             a struct_size that ends before pool_pages means 0 */
  int32_t pool_pages;     /* pool blocks of P rows per sequence (0 with P = 0) */
} skv_tier_desc;

typedef struct {
  int64_t steps;          /* resolve calls */
  int64_t picks;          /* middle positions resolved (sum over sequences) */
  int64_t hits;
  int64_t misses;
  int64_t host_bytes;     /* bytes read from host memory = misses * H_kv * record */
  int64_t in_place;       /* picks read in place from mapped pages; picks = in_place + hits + misses */
} skv_tier_stats;

/* Allocates the tier (device slot state + resident rows; host records unless
 * given).  Host call, synchronous.  SKV_ERR_OOM / SKV_ERR_HOST_MEMORY on failure. */
skv_status sparsekv_tier_create(const skv_tier_desc* d, skv_tier** out);
/* Host pointer of the host records (the caller fills them before resolving);
 * sparsekv_tier_host_ptr is the same call under its other name. */
void* sparsekv_tier_host_records(skv_tier* t);
void* sparsekv_tier_host_ptr(skv_tier* t);
/* Device view of the resident rows. */
skv_status sparsekv_tier_resident(skv_tier* t, skv_kv_view* view);
/* Copies the caller's sink+tail rows ([B][S+L][H_kv][D] int8 and
 * [B][S+L][H_kv] fp16 scales, device) into resident rows [0, S+L). */
skv_status sparsekv_tier_load_resident(skv_tier* t, const int8_t* k, const int8_t* v,
                                       const uint16_t* k_scale, const uint16_t* v_scale,
                                       void* stream);
/* One step, one kernel (the fused resolver of page "vLLM's Hybrid HiSparse
 * ...", section "Three residency states, one block pool"): for each sequence,
 * resolves the selected positions idx[b][0..n_sel) (ascending) -- sinks and
 * tail resident, middle picks of mapped pages in place, the others against
 * the hot buffer (hits refresh their entry, misses take slots) -- reads each
 * missed record from host memory into its slot as int8 rows, and writes
 * rows[b][i] = the resident row of idx[b][i].  The caller then runs
 * sparsekv_tier_attend (or sparsekv_attend on the resident view) with rows,
 * n_sel. */
skv_status sparsekv_tier_resolve(skv_tier* t, const int32_t* idx, const int32_t* n_sel,
                                 int32_t step, int32_t* rows, void* stream);
/* Several query tokens per sequence (a step verifying drafted tokens; page "8
 * agents x 250K ...", which serves with multi-token prediction, and page
 * "vLLM's Hybrid HiSparse ...", which notes that the hot buffer must then hold
 * the rows of every query at once): idx [B][n_query][cap] and n_sel
 * [B][n_query] hold one ascending pick list per query token (e.g. from
 * sparsekv_step_multi), rows [B][n_query][cap] receives the resident row of
 * each pick.  The lists of a sequence are resolved one after another at the
 * same step number, each as by sparsekv_tier_resolve, so the rows an earlier
 * list placed are used in this step: a later list finds them (hits) and
 * cannot evict them, and every row any query needs is resident when the
 * attention (sparsekv_attend_multi on the resident view) runs.  Positions are
 * classified against the tier's context T: a later query's tail positions
 * below T-L are middle rows here.  If the distinct middle rows of the step do
 * not fit the hot buffer, the misses that find no slot get row 0 and
 * SKV_FLAG_TIER_INPUT is raised.  1 <= n_query <= 16. */
skv_status sparsekv_tier_resolve_multi(skv_tier* t, int32_t n_query, const int32_t* idx,
                                       const int32_t* n_sel, int32_t step, int32_t* rows,
                                       void* stream);
/* Attention over the tier's resident rows: sparsekv_attend on the view
 * sparsekv_tier_resident returns, with rows [B][cap] and n_sel from
 * sparsekv_tier_resolve (page "8 agents x 250K ...", section "The mechanism":
 * exact attention on the kept rows, wherever they are resident).  ws as for
 * sparsekv_attend with the tier's layer descriptor. */
skv_status sparsekv_tier_attend(skv_tier* t, const void* q, const int32_t* rows,
                                const int32_t* n_sel, float sm_scale, float* out, void* ws,
                                size_t ws_bytes, void* stream);
/* Page residency.  map_page makes page `page` of sequence `seq` resident in
 * pool block `block` (0 <= block < pool_pages): when k is given, its rows are
 * first copied from device arrays k, v [P][H_kv][D] int8 and k_scale,
 * v_scale [P][H_kv] fp16 (positions page*P .. page*P+P-1, the rows a plain
 * int8 cache holds for them); with k, v, k_scale, v_scale all NULL the block
 * must already hold them.  unmap_page returns the page to host-only (its
 * block becomes free).  Both are enqueued on stream (the next resolve on that
 * stream sees them); SKV_ERR_STATE if the page is already mapped / not
 * mapped or the block is taken; SKV_ERR_INVALID for out-of-range arguments. */
skv_status sparsekv_tier_map_page(skv_tier* t, int32_t seq, int32_t page, int32_t block,
                                  const int8_t* k, const int8_t* v, const uint16_t* k_scale,
                                  const uint16_t* v_scale, void* stream);
skv_status sparsekv_tier_unmap_page(skv_tier* t, int32_t seq, int32_t page, void* stream);
/* Decode-step append for a tier (page "8 agents x 250K ...", section "The
 * mechanism": every token's K/V also goes to host RAM as int4 in 64-dim groups;
 * the GPU keeps the sinks and the recent tail).  For every sequence b the new
 * token goes to position T = ctx_len[b], which must equal the tier's context
 * of b: its host record (group scale g = fp16(fp32(amax/7)), codes
 * clamp(rint(x/g), +-7), K row then V row, as above) is written into host
 * memory through its device address; its int8 rows + fp16 row scales (the
 * rule of sparsekv_append) replace tail position T-L in ring row
 * S + ((T - ctx0) mod L) (none when L = 0); its key sketch is written to
 * index_keys / index_scale row T as by sparsekv_append; then T and ctx_len[b]
 * become T+1.  k_new, v_new: fp16 [B][H_kv][D]; basis fp32 [H_kv][D][R];
 * index_keys [B][max_ctx][H_kv*R/2], index_scale fp16 [B][max_ctx]; ctx_len
 * int32 [B] device, in/out.  A sequence at capacity (T >= max_ctx) or whose
 * ctx_len differs from the tier's context is left unchanged and flagged
 * (SKV_FLAG_CTX_RANGE / SKV_FLAG_TIER_INPUT, reported by sparsekv_tier_stats).
 * Enqueued on stream; calls on one tier must not overlap. */
skv_status sparsekv_tier_append(skv_tier* t, int32_t* ctx_len, const void* k_new,
                                const void* v_new, const float* basis, void* index_keys,
                                uint16_t* index_scale, void* stream);
/* Synchronizes `stream` and returns cumulative counters (host struct). */
skv_status sparsekv_tier_stats(skv_tier* t, skv_tier_stats* out, void* stream);
/* Synchronizes `stream` and copies the slot table to the host:
 * slot_pos [B][n_slots] int32 (position held, -1 empty). */
skv_status sparsekv_tier_slots(skv_tier* t, int32_t* slot_pos_host, void* stream);
/* Empties the hot buffer and zeroes the counters (enqueued on stream). */
skv_status sparsekv_tier_reset(skv_tier* t, void* stream);
void sparsekv_tier_destroy(skv_tier* t);

#ifdef __cplusplus
}
#endif

#endif /* SPARSEKV_H */
