/*
 * attn.h -- C ABI of libattn.so: masked grouped-query attention forward for
 * AMD Instinct MI355X (gfx950), in three forms (prefill over a contiguous KV
 * range, single-query decode over a paged KV cache, DFlash2 block verify).
 *
 * Pages the operations follow (docs.rs source pages):
 *   [prefill] mlx-native 0.18.0, src/ops/flash_attn_prefill_tensor.rs
 *   [paged]   ferrum-kernels 0.8.3, src/backend/metal/vnext_ops/causal_attention.rs
 *   [pack]    mlx-native 0.21.1, src/ops/dflash2_attention_pack.rs
 *
 * Conventions for every entry point:
 *  - Buffer pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains device memory; it keeps no state
 *    between calls beyond its loaded code objects and a thread-local error
 *    string.
 *  - Strides and capacities are in ELEMENTS of the buffer's type, as on the
 *    [prefill] page.  Element types are given by attn_dtype codes.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    work on it and return; the library never synchronises.  Outputs must
 *    not alias inputs, except that dflash_commit updates the ring in place.
 *  - Everything the host can check is checked before anything is enqueued,
 *    as the pages' dispatch functions validate before encoding.  A violation
 *    returns ATTN_EINVAL, enqueues nothing and sets attn_last_error().  A
 *    failed kernel launch returns ATTN_EHIP.
 *  - Values that live in device memory (lengths, positions, counts, page
 *    ids) cannot be checked without a synchronisation.  They are trusted,
 *    but every kernel clamps them to the declared capacities so a bad value
 *    gives a wrong answer, never an out-of-bounds access.
 *  - Base pointers must be 16-byte aligned (128-bit loads).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_OK = 0, ATTN_EINVAL = 1, ATTN_EHIP = 2 } attn_status;
typedef enum { ATTN_NONE = 0, ATTN_F32 = 1, ATTN_F16 = 2, ATTN_BF16 = 3 } attn_dtype;

/* Text of the last non-OK return on the calling thread ("" if none). */
const char *attn_last_error(void);

/* SHA-256 (lowercase hex) of the source files this library was compiled
 * from, so that a loader can tell a stale build from a current one. */
const char *attn_source_sha256(void);

/* KV tile height walked by the kernels: 64 cache rows per step ([prefill],
 * CACHE_ROWS_PER_STEP). */
#define ATTN_KV_TILE 64

/* kv_len rounded up to a multiple of ATTN_KV_TILE ([prefill], kv_pad). */
uint32_t attn_kv_pad(uint32_t kv_len);

/* ------------------------------------------------------------------------
 * Prefill: O = softmax(scale * Q K^T + mask) V per (batch, row, head).
 * [prefill] module header and FlashAttnPrefillTensorParams: Q rows x heads x
 * head_dim with explicit row/head strides, K/V with explicit row/head strides,
 * one KV head per n_heads/n_kv_heads query heads (query head h reads KV head
 * h / (n_heads/n_kv_heads)), an additive mask, O F32.
 *
 * This library generalises the page's contract:
 *  - a batch dimension (stride *_bs) so block verify runs lanes in one call;
 *  - kv_len need not be a multiple of 64: rows >= kv_len are never read and
 *    act as masked (a padded call with -inf columns and an unpadded call
 *    agree);
 *  - the mask may be absent, shared by every head (m_hs = 0, as on the page)
 *    or per head; it is F16 or BF16; columns >= kv_len are not read;
 *  - Q may be F32 or BF16 (the verify path hands over packed bf16 Q);
 *  - head_dim is 128, 256 or 512.
 * Element (b, i, h, d) of Q is q[b*q_bs + i*q_rs + h*q_hs + d]; K row j of KV
 * head kh is k[b*k_bs + j*k_rs + kh*k_hs + d]; mask entry (b, h, i, j) is
 * mask[b*m_bs + h*m_hs + i*m_rs + j]; O is o[b*o_bs + i*o_rs + h*o_hs + d].
 * The *_cap fields give each buffer's size in elements; the largest element
 * the strides address must lie below it ([prefill], need_elems).
 * A row whose keys are all masked yields O = 0.
 * Strides of Q must be multiples of 4 (F32) or 8 (BF16) and strides of K, V
 * multiples of 8 (128-bit loads); O strides multiples of 4.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t batch, rows, kv_len, n_heads, n_kv_heads, head_dim;
    int32_t q_dtype;    /* ATTN_F32 | ATTN_BF16 */
    int32_t kv_dtype;   /* ATTN_F16 | ATTN_BF16 (K and V share it) */
    int32_t mask_dtype; /* ATTN_NONE | ATTN_F16 | ATTN_BF16 */
    float scale;        /* s = scale * (q . k) + mask; the mask is not scaled */
    int64_t q_bs, q_rs, q_hs;
    int64_t k_bs, k_rs, k_hs;
    int64_t v_bs, v_rs, v_hs;
    int64_t m_bs, m_hs, m_rs;
    int64_t o_bs, o_rs, o_hs;
    int64_t q_cap, k_cap, v_cap, m_cap, o_cap;
} attn_prefill_params;

/* Workspace the call needs: a status block, the tile classification of the
 * mask, and partial results when the KV range or a row block is shared by
 * workgroups.  At least ATTN_PREFILL_STATUS_BYTES.  Returns ATTN_OK and writes
 * *bytes, or ATTN_EINVAL for parameters attn_prefill would reject. */
int attn_prefill_workspace_bytes(const attn_prefill_params *p, size_t *bytes);

/* Status block: the first ATTN_PREFILL_STATUS_BYTES of the workspace, as
 * uint32 words, cleared by every call before any other of its kernels run
 * and readable once the call has completed on its stream.
 *   word 0  error flags.  ATTN_PREFILL_WAIT_EXPIRED: a workgroup that merges
 *           a row block it shares with another waited for the other's
 *           partial result past a fixed bound (about 2^22 polls); it wrote
 *           NaN into that row block's output instead of a wrong value.  The
 *           other flags are reserved and stay 0.
 *   word 1  row blocks whose key range two workgroups shared and merged
 *           (diagnostic: how often that merge ran; 0 for calls without a mask).
 * The other words are reserved. */
#define ATTN_PREFILL_STATUS_BYTES 256
#define ATTN_PREFILL_WAIT_EXPIRED 1u

/* q, k, v, mask: device inputs as described above (mask may be NULL iff
 * mask_dtype == ATTN_NONE); o: device output; ws: device workspace of at
 * least attn_prefill_workspace_bytes() bytes, 16-byte aligned. */
int attn_prefill(const attn_prefill_params *p, const void *q, const void *k, const void *v,
                 const void *mask, float *o, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Paged decode: one query per sequence against its whole context, read
 * through a page table ([paged]: pages of a fixed number of tokens, per-token
 * K and V rows of n_kv_heads x head_dim, the context of a step includes the
 * token it just wrote, query head h reads KV head h / (n_heads/n_kv_heads)).
 * Token t of sequence b is in pool page page_table[b*max_pages_per_seq +
 * t/page_size], slot t % page_size; its K row for KV head kh starts at
 *   page*kv_page_stride + slot*kv_token_stride + kh*kv_head_stride
 * in k_pool (and likewise in v_pool, which shares the strides; the page's
 * interleaved [2, kv_heads, head_dim] token record is k_pool = base,
 * v_pool = base + kv_heads*head_dim, kv_token_stride = 2*kv_heads*head_dim).
 * context_lens[b] is clamped to [0, min(max_context, max_pages_per_seq *
 * page_size)]; page ids are clamped to [0, num_pages); entries of the page
 * table past the context are never read.  A sequence with an empty context
 * yields O = 0.  Q, O: F32 [batch, n_heads, head_dim] with strides
 * (q_bs, q_hs), (o_bs, o_hs).  head_dim is 128 or 256 ([paged]: at most 256).
 * kv_cap is the size of each pool in elements.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t batch, n_heads, n_kv_heads, head_dim;
    int32_t page_size, max_pages_per_seq, num_pages, max_context;
    int32_t kv_dtype; /* ATTN_F16 | ATTN_BF16 */
    float scale;
    int64_t q_bs, q_hs, o_bs, o_hs;
    int64_t kv_page_stride, kv_token_stride, kv_head_stride;
    int64_t q_cap, kv_cap, o_cap;
} attn_decode_params;

int attn_paged_decode_workspace_bytes(const attn_decode_params *p, size_t *bytes);

int attn_paged_decode(const attn_decode_params *p, const float *q, const void *k_pool,
                      const void *v_pool, const int32_t *page_table, const int32_t *context_lens,
                      float *o, void *ws, size_t ws_bytes, void *stream);

/* Paged decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Arguments and results are attn_paged_decode's; the
 * split partials live instead in a static device array of
 * ATTN_DECODE_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call allocates and frees nothing.  It returns
 * ATTN_EINVAL, enqueueing nothing, when attn_paged_decode_workspace_bytes for
 * the same parameters exceeds ATTN_DECODE_SCRATCH_BYTES (the paged workload of
 * 64 sequences of up to 16384 tokens, 32 heads, head_dim 128, needs 34.6 MB),
 * and ATTN_EHIP if the array's address cannot be found for the current device.
 * Every call on one GPU shares that GPU's array: calls that may run at the
 * same time on one GPU (unordered streams) race and give wrong results. */
#define ATTN_DECODE_SCRATCH_BYTES (64u << 20)
int attn_paged_decode_noalloc(const attn_decode_params *p, const float *q, const void *k_pool,
                              const void *v_pool, const int32_t *page_table,
                              const int32_t *context_lens, float *o, void *stream);

/* ------------------------------------------------------------------------
 * Multi-token paged attention ([paged]: `tokens` new tokens from
 * `position_start`, causal, over the same paged KV layout as decode; the
 * new tokens' K/V rows are already in the pages).  Query token i of sequence
 * b (i < query_lens[b] <= max_tokens) sits at position s = position_starts[b]
 * + i and attends to the keys t <= s of its sequence:
 *   O[b,i,h,:] = softmax_t(scale * Q[b,i,h,:] . K[b,t,h/g,:]) . V[b,t,h/g,:]
 * With one token at position context - 1 it is the decode step; with more
 * it is chunked prefill (at most 64 tokens per sequence per call) or block
 * verify straight from the page table.
 * Page addressing, clamping and pool strides as attn_paged_decode; the
 * context of sequence b is position_starts[b] + query_lens[b], both clamped
 * (starts to [0, cap], lengths to [0, max_tokens], the context to cap =
 * min(max_context, max_pages_per_seq * page_size)); page-table entries past
 * it are never read.  Q, O: F32 [batch, max_tokens, n_heads, head_dim] with
 * strides (q_bs, q_ts, q_hs), (o_bs, o_ts, o_hs); rows i >= query_lens[b]
 * of O are not written.  head_dim 128 or 256; 1 <= max_tokens <= 64.
 * ws: caller-owned device workspace of attn_paged_prefill_workspace_bytes
 * bytes, 16-byte aligned; its contents need no initialisation.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t batch, n_heads, n_kv_heads, head_dim;
    int32_t page_size, max_pages_per_seq, num_pages, max_context, max_tokens;
    int32_t kv_dtype; /* ATTN_F16 | ATTN_BF16 */
    float scale;
    int64_t q_bs, q_ts, q_hs, o_bs, o_ts, o_hs;
    int64_t kv_page_stride, kv_token_stride, kv_head_stride;
    int64_t q_cap, kv_cap, o_cap;
} attn_paged_prefill_params;

int attn_paged_prefill_workspace_bytes(const attn_paged_prefill_params *p, size_t *bytes);

int attn_paged_prefill(const attn_paged_prefill_params *p, const float *q, const void *k_pool,
                       const void *v_pool, const int32_t *page_table, const int32_t *query_lens,
                       const int32_t *position_starts, float *o, void *ws, size_t ws_bytes,
                       void *stream);

/* ------------------------------------------------------------------------
 * Prepare ([paged], the prepare dispatch before attention): for token t <
 * query_lens[b] of sequence b, at position s = position_starts[b] + t,
 *  - Q and K heads: RMS norm over the head's head_dim features,
 *      x / sqrt(mean(x^2) + epsilon) * w   (w: the head's norm weights;
 *      qn_hs / kn_hs = 0 shares one vector across heads), skipped if
 *      qk_norm = 0; then rotary embedding of the first rope_dim features,
 *      pair i rotated by s * rope_theta^(-2i/rope_dim), pairs (2i, 2i+1)
 *      if rope_interleaved else (i, i + rope_dim/2); the rest pass through;
 *  - V heads: unchanged;
 *  - prepared Q -> q_out (F32, ready for attn_paged_prefill), K and V ->
 *    their pools (F16/BF16, rounded to nearest even) at page
 *    page_table[b][s / page_size], slot s % page_size (positions at or past
 *    min(max_context, max_pages_per_seq * page_size) are not written).
 * Raw projections are F32 [batch, max_tokens, heads, >= head_dim] with
 * strides (bs, ts, hs); a query head stride of 2*head_dim leaves an output
 * gate half untouched.  Norm weights are F32.  head_dim 128 or 256;
 * 0 < rope_dim <= head_dim, rope_dim even ([paged] shape rules).  Rows are
 * read and written 16 bytes at a time: the F32 buffers 16-byte aligned, the
 * pools 8-byte aligned, every stride a multiple of 4 elements (ATTN_EINVAL
 * otherwise).
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t batch, n_heads, n_kv_heads, head_dim, max_tokens;
    int32_t rope_dim, rope_interleaved, qk_norm;
    int32_t page_size, max_pages_per_seq, num_pages, max_context;
    int32_t kv_dtype; /* ATTN_F16 | ATTN_BF16 */
    float epsilon, rope_theta;
    int64_t qr_bs, qr_ts, qr_hs, kr_bs, kr_ts, kr_hs, vr_bs, vr_ts, vr_hs;
    int64_t qo_bs, qo_ts, qo_hs;
    int64_t qn_hs, kn_hs;
    int64_t kv_page_stride, kv_token_stride, kv_head_stride;
    int64_t qr_cap, kr_cap, vr_cap, qo_cap, qn_cap, kn_cap, kv_cap;
} attn_paged_prepare_params;

int attn_paged_prepare(const attn_paged_prepare_params *p, const float *q_raw, const float *k_raw,
                       const float *v_raw, const float *q_norm, const float *k_norm,
                       const int32_t *page_table, const int32_t *query_lens,
                       const int32_t *position_starts, float *q_out, void *k_pool, void *v_pool,
                       void *stream);

/* ------------------------------------------------------------------------
 * DFlash2 block verify ([pack]).  Geometry as DFlash2AttentionPackParams with
 * the same rules ([pack], validate): 1 <= lanes <= 4; heads > 0; q_heads a
 * multiple of kv_heads; head_dim 128 or 256; 2 <= rows <= 16; window > rows;
 * packed_len == window - 1 + rows; 1 <= max_commit <= rows.
 * Buffers are contiguous with exactly the shapes the page's dispatch
 * functions require, and each call takes the byte length of every buffer,
 * which must equal the shape's ([pack], require):
 *   ring K/V        bf16 [lanes, kv_heads, window, head_dim]
 *   current Q       f32  [lanes, rows, q_heads, head_dim]
 *   current K/V     f32  [lanes, rows, kv_heads, head_dim]
 *   cache lengths, write positions, commit counts   u32 [lanes]
 *   packed Q        bf16 [lanes, q_heads, rows, head_dim]
 *   packed K/V      bf16 [lanes, kv_heads, packed_len, head_dim]
 *   mask            bf16 [lanes, q_heads, rows, packed_len]
 *   new K/V         f32  [lanes, max_commit, kv_heads, head_dim]
 * f32 -> bf16 conversion rounds to nearest even (NaN stays NaN).
 * ---------------------------------------------------------------------- */
typedef struct {
    uint32_t lanes, q_heads, kv_heads, head_dim, rows, window, packed_len, max_commit;
} dflash_params;

/* Host-side geometry check alone ([pack], validate): ATTN_OK or ATTN_EINVAL. */
int dflash_validate(const dflash_params *p);

/* Pack: packed Q[b,h,i,:] = bf16(current Q[b,i,h,:]); packed K/V position
 * p < rows holds bf16 of drafted row p; position rows + j holds ring slot
 * (write_position - 1 - j) mod window (newest first) while j < cache_length,
 * else zero.  bytes[10] = byte lengths of ring_k, ring_v, cur_q, cur_k,
 * cur_v, cache_lengths, write_positions, packed_q, packed_k, packed_v. */
int dflash_pack(const dflash_params *p, const uint16_t *ring_k, const uint16_t *ring_v,
                const float *cur_q, const float *cur_k, const float *cur_v,
                const uint32_t *cache_lengths, const uint32_t *write_positions,
                uint16_t *packed_q, uint16_t *packed_k, uint16_t *packed_v,
                const uint64_t *bytes, void *stream);

/* Mask: mask[b,h,i,p] = 0 if p < rows or p - rows < min(cache_length,
 * window - 1 - i), else -inf (bf16 0xFF80); the same for every head.
 * bytes[2] = byte lengths of cache_lengths, mask. */
int dflash_mask(const dflash_params *p, const uint32_t *cache_lengths, uint16_t *mask,
                const uint64_t *bytes, void *stream);

/* Commit: for c < min(commit_count, max_commit), ring row (write_position + c)
 * mod window = bf16(new row c), for K and V, in place.  Neither the cache
 * length nor the write position is read or advanced here (the caller moves
 * them by the committed count).  bytes[6] = byte lengths of new_k, new_v,
 * commit_counts, write_positions, ring_k, ring_v. */
int dflash_commit(const dflash_params *p, const float *new_k, const float *new_v,
                  const uint32_t *commit_counts, const uint32_t *write_positions,
                  uint16_t *ring_k, uint16_t *ring_v, const uint64_t *bytes, void *stream);

/* Pack-free verify attention: the attention that pack, mask and a masked GQA
 * attention over the packed buffers compute ([pack], the pack and mask
 * kernels' key order and visibility rule), read from the ring in place.
 * For lane b with cache length L and write position wp, query row i of head
 * h attends over (1) the drafted rows p < rows, bf16 of current K/V row p,
 * all visible, then (2) ring slot (wp - 1 - j) mod window for
 * j < min(L, window - 1 - i), newest first:
 *   out[b,h,i,:] = softmax_j(scale * bf16(cur_q[b,i,h,:]) . k_j) . v_j
 * with KV head h / (q_heads / kv_heads); out f32 [lanes, q_heads, rows,
 * head_dim], contiguous.  Ring slots outside a lane's visible range are
 * never read.  Geometry as dflash_validate, plus window <= 2^24.
 * ws: caller-owned device workspace of dflash_verify_workspace_bytes bytes
 * (split partials), 16-byte aligned; its contents need no initialisation.
 * bytes[8] = byte lengths of ring_k, ring_v, cur_q, cur_k, cur_v,
 * cache_lengths, write_positions, out.  Asynchronous on `stream`. */
int dflash_verify_workspace_bytes(const dflash_params *p, size_t *bytes);
int dflash_verify_attention(const dflash_params *p, float scale, const uint16_t *ring_k,
                            const uint16_t *ring_v, const float *cur_q, const float *cur_k,
                            const float *cur_v, const uint32_t *cache_lengths,
                            const uint32_t *write_positions, float *out, void *ws, size_t ws_bytes,
                            const uint64_t *bytes, void *stream);

/* Mask rows ([pack], the mask-rows kernel): rows 1..rows-1 of every lane's
 * f32 draft input [lanes*rows, hidden] become the bf16 mask embedding
 * [hidden] widened to f32; row 0 (the anchor) is kept.  Rules ([pack]):
 * 1 <= lanes <= 4, 2 <= rows <= 16, hidden > 0.  bytes[2] = byte lengths of
 * mask_embedding, draft_input. */
int dflash_mask_rows(uint32_t lanes, uint32_t rows, uint32_t hidden, const uint16_t *mask_embedding,
                     float *draft_input, const uint64_t *bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
