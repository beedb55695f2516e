/*
 * kb_attn -- bitwise-aligned causal grouped-query attention for AMD
 * Instinct MI355X (gfx950): the forward entry points, and a deterministic
 * backward.
 *
 * The operator is the unified attention of the KernelBraid / AReaL-TIK README:
 *   - "Features": BF16, causal, contiguous [batch, heads, sequence, head_dim]
 *     tensors, 32 query heads, 8 KV heads, head_dim 128;
 *   - "Usage": two calls, unified_prefill (the whole causal sequence) and
 *     unified_decode (the last token against all cached keys); the decoded
 *     row and the prefill's last row are compared as raw bf16 bits, and each
 *     result takes q's shape;
 *   - "Method" / "Advantages": prefill, the chunked (partitioned) forward and
 *     one-token decode follow one set of numerical rules, which is what makes
 *     their results for a given row and context the same bit pattern.
 *
 * Numerical contract (shared by every entry point): for the query row at
 * absolute position pos (keys 0..pos visible, KV head = q head / 4),
 * keys are visited in tiles of KB_ATTN_KV_TILE keys from key 0 and grouped in
 * chunks of KB_ATTN_KV_CHUNK keys; each chunk runs an fp32 online softmax over
 * its tiles in order, and chunk results are folded in chunk order.  The output
 * bits depend only on (q row, K/V rows 0..pos, scale).
 *
 * Conventions for every entry point:
 *   - q, k, v, o, k_cache, v_cache are DEVICE pointers of the current HIP
 *     device to bf16 values (raw 16-bit patterns), 16-byte aligned.
 *   - q and o are [batch, n_q_heads, q_len, head_dim] contiguous.
 *   - k/v (prefill) are [batch, n_kv_heads, seq_len, head_dim] contiguous;
 *     k_cache/v_cache are [batch, n_kv_heads, kv_capacity, head_dim]
 *     contiguous, of which rows 0..kv_len-1 are read (the caller writes the
 *     current token(s) before the call; the library never writes the cache).
 *   - head_dim must be 128 and n_q_heads must equal 4 * n_kv_heads.
 *   - scale multiplies <q, k>; it must be finite and > 0 (1/sqrt(128) in the
 *     README's workloads, whose API takes no scale).
 *   - q, k and v must hold finite values.  Scores are accumulated in fp32, so
 *     a row whose scale * <q, k_j> leaves the fp32 range (about 3.4e38) is
 *     outside the contract and its output is not specified; the library does
 *     not check the values (that would cost a pass over the cache).  The
 *     softmax weights are kept relative to a reference maximum that may lag
 *     the true one by up to 2^64, so a row's running sums reach at most
 *     kv_len * 2^64 and kv_len * 2^64 * max|v|; the contract also needs
 *     kv_len * max|v| < 2^64 (|v| < 2^34 at the longest kv_len, 2^30).
 *   - The caller owns every buffer; the library allocates nothing, keeps no
 *     state (except kb_attn_decode_static's per-GPU scratch, below) and is
 *     thread-safe (kb_attn_decode_static calls that overlap on one GPU race
 *     on that scratch).  Calls are asynchronous on `stream` (0 = the null
 *     stream) and return once the work is enqueued.
 *   - o must not overlap any input.
 *   - Every argument is checked before anything is launched; on error nothing
 *     is launched and a negative KB_ATTN_ERR_* code is returned.
 */
#ifndef KB_ATTN_H
#define KB_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KB_ATTN_KV_TILE 64
#define KB_ATTN_KV_CHUNK 1024
#define KB_ATTN_CONTRACT_VERSION 6

enum {
    KB_ATTN_OK = 0,
    KB_ATTN_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, bad scale */
    KB_ATTN_ERR_UNSUPPORTED = -2, /* head_dim != 128 or n_q_heads != 4 * n_kv_heads */
    KB_ATTN_ERR_LENGTH = -3,      /* q_len < 1, q_len > kv_len or kv_len > kv_capacity */
    KB_ATTN_ERR_ALIGNMENT = -4,   /* a pointer is not 16-byte aligned */
    KB_ATTN_ERR_DEVICE = -5,      /* a pointer is not device memory of the current device */
    KB_ATTN_ERR_WORKSPACE = -6,   /* decode workspace missing or too small */
    KB_ATTN_ERR_ALIAS = -7,       /* the output overlaps an input or the workspace */
    KB_ATTN_ERR_HIP = -8,         /* a HIP call or kernel launch failed */
    KB_ATTN_ERR_SCRATCH = -9      /* the call needs more than the library's static scratch */
};

/*
 * Causal full-sequence forward ("Usage": unified_prefill).  Query row r sits
 * at position r and attends to keys 0..r of KV head h / 4.
 * q, o: [batch, n_q_heads, seq_len, 128]; k, v: [batch, n_kv_heads, seq_len, 128].
 */
int kb_attn_prefill(const void* q, const void* k, const void* v, void* o, int64_t batch,
                    int64_t seq_len, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                    float scale, hipStream_t stream);

/*
 * Partitioned (chunked) forward ("Method": partitioned forward execution;
 * "Usage": prompt/answer splits).  A chunk of q_len query rows against a
 * cache holding kv_len keys; row r sits at position kv_len - q_len + r
 * (bottom-right causal), so a sequence cut into chunks reproduces the prefill
 * rows bit for bit.
 * q, o: [batch, n_q_heads, q_len, 128]; caches: [batch, n_kv_heads, kv_capacity, 128].
 */
int kb_attn_partitioned(const void* q, const void* k_cache, const void* v_cache, void* o,
                        int64_t batch, int64_t q_len, int64_t kv_len, int64_t kv_capacity,
                        int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                        hipStream_t stream);

/*
 * One-token decode ("Usage": unified_decode over the full KV context).  The
 * single query row sits at position kv_len - 1.  When kv_len exceeds one
 * chunk the keys are split by chunk across workgroups; the partial results go
 * to `workspace` (fp32, caller owned, at least
 * kb_attn_decode_workspace_bytes(...) bytes, device memory) and are folded in
 * chunk order, the same order the prefill kernel uses.  workspace may be
 * NULL when that size is 0.  Concurrent calls need separate workspaces.
 * q, o: [batch, n_q_heads, 1, 128]; caches: [batch, n_kv_heads, kv_capacity, 128].
 */
int kb_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, int64_t batch,
                   int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads,
                   int32_t head_dim, float scale, void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/* Workspace bytes kb_attn_decode needs (0 when kv_len fits in one chunk;
 * 0 for invalid sizes). */
size_t kb_attn_decode_workspace_bytes(int64_t batch, int64_t kv_len, int32_t n_q_heads,
                                      int32_t head_dim);

/* Size of the scratch array behind kb_attn_decode_static (8 MiB). */
#define KB_ATTN_DECODE_STATIC_SCRATCH_BYTES (8u << 20)

/*
 * kb_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The chunk partials go to a scratch array
 * the library keeps in device memory, one copy per GPU it runs on, held until
 * the process ends; the first call on a device looks up that device's copy.
 * The call allocates nothing.  A call that needs more than
 * KB_ATTN_DECODE_STATIC_SCRATCH_BYTES (kb_attn_decode_workspace_bytes(...) of
 * the same sizes; B * n_q_heads * ceil(kv_len / 1024) <= 16131 partial rows,
 * e.g. batch 16 with 32 heads up to 31744 keys) returns KB_ATTN_ERR_SCRATCH
 * and launches nothing.  Every call on one GPU shares the array and it keeps
 * the last call's contents (no call depends on them: each partial is written
 * before it is read): calls whose work may overlap on one GPU (several
 * streams, several host threads) race and must be serialised by the caller.
 * Output bits are those of kb_attn_decode.  Other arguments and rules as for
 * kb_attn_decode.
 */
int kb_attn_decode_static(const void* q, const void* k_cache, const void* v_cache, void* o,
                          int64_t batch, int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads,
                          int32_t n_kv_heads, int32_t head_dim, float scale, hipStream_t stream);

/*
 * Decode of the last n_rows tokens (1 <= n_rows <= 8, else
 * KB_ATTN_ERR_UNSUPPORTED), e.g. several drafted tokens checked at once: the
 * partitioned forward of a short chunk ("Method": partitioned forward
 * execution), run with decode's split over 1024-key chunks.  Row r of each
 * head sits at position kv_len - n_rows + r (n_rows <= kv_len <= kv_capacity,
 * else KB_ATTN_ERR_LENGTH), and its bits equal those of the prefill row at
 * that position (a row takes part only in the chunks up to the one holding
 * its position).
 * q, o: [batch, n_q_heads, n_rows, 128]; caches as kb_attn_decode; workspace
 * as kb_attn_decode, sized by kb_attn_decode_multi_workspace_bytes.
 */
int kb_attn_decode_multi(const void* q, const void* k_cache, const void* v_cache, void* o,
                         int64_t batch, int64_t n_rows, int64_t kv_len, int64_t kv_capacity,
                         int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes kb_attn_decode_multi needs (0 when kv_len fits in one
 * chunk; 0 for invalid sizes). */
size_t kb_attn_decode_multi_workspace_bytes(int64_t batch, int64_t n_rows, int64_t kv_len,
                                            int32_t n_q_heads, int32_t head_dim);

/*
 * Ragged (variable-length) batches of the three entry points: the same
 * contract, row by row, so a sequence's outputs are bit for bit those of the
 * dense call on that sequence alone.  (Rollout batches mix prompt and answer
 * lengths; the "Usage" section's prompt/answer splits are per sequence.)
 *
 * Packed layout, head-major: a tensor with H heads and R rows per head is
 * [H, R, 128] contiguous, and sequence i owns rows off[i] .. off[i+1] - 1 of
 * every head.  The offset and length arrays are HOST arrays (batch + 1
 * offsets, non-decreasing from >= 0; batch lengths); they are read during the
 * call, checked in full before anything is launched, and not kept.  Sequences
 * with no query rows are skipped.  Any batch size is accepted; the work is
 * issued in launches of at most 64 sequences.
 */

/* Causal prefill of every sequence: q, o [n_q_heads, cu_seqlens[batch], 128];
 * k, v [n_kv_heads, cu_seqlens[batch], 128]; row r of sequence i sits at
 * position r of that sequence. */
int kb_attn_prefill_varlen(const void* q, const void* k, const void* v, void* o,
                           const int64_t* cu_seqlens, int64_t batch, int32_t n_q_heads,
                           int32_t n_kv_heads, int32_t head_dim, float scale, hipStream_t stream);

/* Partitioned forward of every sequence: q, o [n_q_heads, cu_q[batch], 128];
 * caches [n_kv_heads, cu_cache[batch], 128].  Sequence i has
 * q_len = cu_q[i+1] - cu_q[i] query rows, a cache range of capacity
 * cu_cache[i+1] - cu_cache[i] rows of which the first kv_lens[i] are keys
 * (0 <= q_len <= kv_len <= capacity, else KB_ATTN_ERR_LENGTH); its row r sits
 * at position kv_lens[i] - q_len + r. */
int kb_attn_partitioned_varlen(const void* q, const void* k_cache, const void* v_cache, void* o,
                               const int64_t* cu_q, const int64_t* cu_cache,
                               const int64_t* kv_lens, int64_t batch, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, float scale,
                               hipStream_t stream);

/* One-token decode of every sequence: q, o [n_q_heads, batch, 128] (one row
 * per sequence); caches as in kb_attn_partitioned_varlen, with
 * 1 <= kv_lens[i] <= capacity.  Sequences longer than one chunk are split by
 * chunk; their partials go to `workspace` (device memory, at least
 * kb_attn_decode_varlen_workspace_bytes(kv_lens, ...) bytes; NULL when that
 * is 0) and are folded in chunk order. */
int kb_attn_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* o,
                          const int64_t* cu_cache, const int64_t* kv_lens, int64_t batch,
                          int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes kb_attn_decode_varlen needs for these host kv_lens (0 when
 * no sequence exceeds one chunk; 0 for invalid arguments). */
size_t kb_attn_decode_varlen_workspace_bytes(const int64_t* kv_lens, int64_t batch,
                                             int32_t n_q_heads, int32_t head_dim);

/*
 * One-token decode over a paged KV cache, the layout rollout engines keep
 * (an extension the pages leave open: "Method" lets data movement vary
 * inside the contract).  Output bits equal those of kb_attn_decode on the
 * same keys laid out contiguously.
 *   q, o         [batch, n_q_heads, 128] (DEVICE, as kb_attn_decode's q, o)
 *   k_pages,
 *   v_pages      page pools [n_pages, n_kv_heads, page_size, 128] (DEVICE);
 *                page_size must be a multiple of 64 (KB_ATTN_ERR_UNSUPPORTED),
 *                so every 64-key tile lies inside one page
 *   block_table  int32 [batch, max_pages] (DEVICE, 4-byte aligned): key j of
 *                sequence i is row j % page_size of page
 *                block_table[i * max_pages + j / page_size]; entries outside
 *                [0, n_pages) are clamped into the pool (no access leaves it;
 *                the output of such a sequence is then unspecified)
 *   kv_lens      HOST int64 [batch], 1 <= kv_lens[i] <= max_pages * page_size
 *   workspace    as kb_attn_decode_varlen (size it with
 *                kb_attn_decode_varlen_workspace_bytes(kv_lens, ...)).
 */
int kb_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o,
                         const int32_t* block_table, int64_t max_pages, const int64_t* kv_lens,
                         int64_t batch, int64_t n_pages, int32_t page_size, int32_t n_q_heads,
                         int32_t n_kv_heads, int32_t head_dim, float scale, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * The three dense entry points with a log-sum-exp output, for a backward
 * pass (README "Background": training forward and backward still run beside
 * the rollout; the pages define no backward, so this one is an extension).
 * Arguments and outputs as in the plain call, plus
 *   lse  fp32 [batch, n_q_heads, rows] (rows = seq_len, q_len or 1; DEVICE,
 *        4-byte aligned, overlapping no other buffer, else
 *        KB_ATTN_ERR_ALIGNMENT / KB_ATTN_ERR_ALIAS; NULL is
 *        KB_ATTN_ERR_INVALID_ARG): log(sum_j exp(scale <q, k_j>)) over the
 *        row's visible keys, computed from the contract's final fp32 state
 *        (Mc, L) as (Mc + log2 L) * ln 2.
 * The output bits o are those of the plain call, and the lse of a row is, like
 * o, bit for bit the same from all three entry points.
 */
int kb_attn_prefill_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t batch, int64_t seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, float scale, hipStream_t stream);
int kb_attn_partitioned_lse(const void* q, const void* k_cache, const void* v_cache, void* o,
                            float* lse, int64_t batch, int64_t q_len, int64_t kv_len,
                            int64_t kv_capacity, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, float scale, hipStream_t stream);
int kb_attn_decode_lse(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                       int64_t batch, int64_t kv_len, int64_t kv_capacity, int32_t n_q_heads,
                       int32_t n_kv_heads, int32_t head_dim, float scale, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of the causal full-sequence forward (an extension: the pages
 * cover the forward only, README "Features" and "Background").  For the
 * upstream gradient dout of o = attention(q, k, v):
 *   dv_j = sum_i P_ij dout_i,   dS_ij = P_ij (<dout_i, v_j> - D_i),
 *   D_i  = <dout_i, o_i>,  dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i
 * with P_ij = exp(scale <q_i, k_j> - lse_i) recomputed in fp32 from the lse
 * a *_lse forward returned, P and dS rounded to bf16 for the products (fp32
 * accumulation), and dk, dv summed over the 4 query heads of each KV head.
 * No atomics: every output element is reduced in one fixed order, so the
 * result bits depend only on the inputs (not on the batch they share, the
 * launch or the run).
 *   q, o, dout, dq  [batch, n_q_heads, seq_len, 128] bf16 (DEVICE, 16-byte aligned)
 *   k, v, dk, dv    [batch, n_kv_heads, seq_len, 128] bf16
 *   lse             fp32 [batch, n_q_heads, seq_len] (DEVICE, 4-byte aligned)
 *   workspace       DEVICE, 16-byte aligned, at least
 *                   kb_attn_backward_workspace_bytes(...) bytes (per-row D_i
 *                   and lse in log2 units); concurrent calls need separate ones
 * dq, dk, dv must not overlap each other, any input or the workspace
 * (KB_ATTN_ERR_ALIAS).  Other errors as for kb_attn_prefill.
 */
int kb_attn_backward(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int64_t batch, int64_t seq_len,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes kb_attn_backward needs (0 for invalid sizes). */
size_t kb_attn_backward_workspace_bytes(int64_t batch, int64_t seq_len, int32_t n_q_heads,
                                        int32_t head_dim);

/*
 * Ragged batches for training (README "Background": the rollout batches the
 * forward serves are ragged, and the policy update runs on the same
 * sequences), in the packed head-major layout of the ragged forward calls:
 *   kb_attn_prefill_varlen_lse   kb_attn_prefill_varlen plus lse fp32
 *                                [n_q_heads, cu_seqlens[batch]] (DEVICE,
 *                                4-byte aligned, overlapping nothing else);
 *                                each row's lse bits equal those of the dense
 *                                prefill_lse of its sequence alone
 *   kb_attn_backward_varlen      kb_attn_backward for every sequence of the
 *                                batch: q, o, dout, dq [n_q_heads, T, 128],
 *                                k, v, dk, dv [n_kv_heads, T, 128], lse
 *                                [n_q_heads, T], T = cu_seqlens[batch];
 *                                sequence i is rows cu_seqlens[i] ..
 *                                cu_seqlens[i+1] - 1 of every head (full
 *                                causal, positions 0 .. len - 1); its
 *                                gradient bits equal those of the dense
 *                                backward of that sequence alone
 * cu_seqlens is a HOST array of batch + 1 non-decreasing offsets from >= 0
 * (each sequence at most 2^30 rows, else KB_ATTN_ERR_LENGTH), read during the
 * call and not kept; empty sequences are skipped.  The backward's workspace
 * (DEVICE, 16-byte aligned; NULL when its size is 0) holds each sequence's
 * rows padded to a multiple of 64.  Other rules as for the dense calls.
 */
int kb_attn_prefill_varlen_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                               const int64_t* cu_seqlens, int64_t batch, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, float scale, hipStream_t stream);
int kb_attn_backward_varlen(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            const int64_t* cu_seqlens, int64_t batch, int32_t n_q_heads,
                            int32_t n_kv_heads, int32_t head_dim, float scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes kb_attn_backward_varlen needs for these host offsets (0
 * when every sequence is empty or the offsets are invalid). */
size_t kb_attn_backward_varlen_workspace_bytes(const int64_t* cu_seqlens, int64_t batch,
                                               int32_t n_q_heads, int32_t head_dim);

/* Static description of an error code (never NULL). */
const char* kb_attn_strerror(int code);

/* The contract constants compiled into the library (any pointer may be NULL). */
void kb_attn_contract(int32_t* kv_tile, int32_t* kv_chunk, int32_t* version);

#ifdef __cplusplus
}
#endif

#endif /* KB_ATTN_H */
