/*
 * oracle.c -- plain, slow, fp64 CPU reference for the masked grouped-query
 * attention forward and the DFlash2 ring pack / mask / commit steps.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code with the HIP kernels.
 *
 * Sources (docs.rs source pages):
 *   [pack]    mlx-native 0.21.1, src/ops/dflash2_attention_pack.rs
 *   [prefill] mlx-native 0.18.0, src/ops/flash_attn_prefill_tensor.rs
 *   [paged]   ferrum-kernels 0.8.3, src/backend/metal/vnext_ops/causal_attention.rs
 *
 * Every floating-point input is widened exactly to double (f32, f16 and bf16
 * all embed exactly in fp64) and all arithmetic is done in double.
 *
 * Pins (see tests/test_oracle_*.py): closed forms, invariants, a float64
 * library SDPA cross-check, the worked examples printed on the [pack] page,
 * brute force over tiny ring geometries, and a library f32->bf16 cast.
 * One convention is parity unpinned by the pages: the value written to
 * packed cache slots at or beyond the cache length (zero here); see
 * oracle_dflash_pack.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Element type codes for the loaders below. */
enum { ORC_F64 = 0, ORC_F32 = 1, ORC_F16 = 2, ORC_BF16 = 3 };

/* ---------------------------------------------------------------------------
 * Exact widening of 16-bit floats.
 * IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * bfloat16: the top 16 bits of an IEEE binary32.
 * ------------------------------------------------------------------------- */
double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exponent = (h >> 10) & 0x1f;
    int fraction = h & 0x3ff;
    double magnitude;
    if (exponent == 0) {
        magnitude = ldexp((double)fraction, -24); /* subnormal: f * 2^-14 / 2^10 */
    } else if (exponent == 31) {
        magnitude = fraction ? NAN : INFINITY;
    } else {
        magnitude = ldexp((double)(1024 + fraction), exponent - 25);
    }
    return sign ? -magnitude : magnitude;
}

double oracle_bf16_to_f64(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int dtype, int64_t index) {
    switch (dtype) {
    case ORC_F64: return ((const double *)base)[index];
    case ORC_F32: return (double)((const float *)base)[index];
    case ORC_F16: return oracle_f16_to_f64(((const uint16_t *)base)[index]);
    case ORC_BF16: return oracle_bf16_to_f64(((const uint16_t *)base)[index]);
    default: return NAN;
    }
}

/* ---------------------------------------------------------------------------
 * f32 -> bf16, round to nearest, ties to even, on the f32 bit pattern.
 * [pack] stores bf16 everywhere and converts the f32 current rows on the way
 * in (kernel table and the commit step); the page's test helper only ever
 * converts exactly representable values, so the rounding rule is a reading:
 * nearest-even, NaN kept NaN (quiet bit set), overflow rounds to infinity,
 * subnormals kept.
 * ------------------------------------------------------------------------- */
uint16_t oracle_bf16_from_f32(float x) {
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    if ((bits & 0x7fffffffu) > 0x7f800000u) {           /* NaN */
        return (uint16_t)((bits >> 16) | 0x0040u);
    }
    uint32_t upper = bits >> 16;
    uint32_t lower = bits & 0xffffu;
    /* round up when the dropped half is above one half, or exactly one half
     * and the kept part is odd */
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) {
        upper += 1u;                                     /* may carry into the exponent */
    }
    return (uint16_t)upper;
}

void oracle_bf16_from_f32_array(const float *x, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_from_f32(x[i]);
}

/* ---------------------------------------------------------------------------
 * One output row of softmax attention, written out as the definition:
 *   s_j = scale * <q, k_j> + mask_j          (mask_j = 0 when absent)
 *   m   = max_j s_j;   if m = -inf the row sees nothing and O = 0
 *   p_j = exp(s_j - m),  l = sum_j p_j,  O = sum_j p_j v_j / l
 * [prefill] module header: additive mask, scale folded into Q ("pre-softmax
 * scale"), one KV head per n_heads/n_kv_heads query heads.
 * `s` is caller scratch of n_keys doubles.
 * ------------------------------------------------------------------------- */
typedef struct {
    const void *base;
    int dtype;
} elem_ref;

static void attend_row(int64_t n_keys, int64_t head_dim, double scale,
                       const double *q,                  /* [head_dim] */
                       elem_ref k, const int64_t *k_off, /* row j starts at k_off[j] */
                       elem_ref v, const int64_t *v_off,
                       elem_ref mask, int64_t mask_off, int64_t mask_step, int has_mask,
                       double *s, double *out /* [head_dim] */) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < head_dim; ++d) dot += q[d] * load_elem(k.base, k.dtype, k_off[j] + d);
        double sj = scale * dot;
        if (has_mask) sj += load_elem(mask.base, mask.dtype, mask_off + j * mask_step);
        s[j] = sj;
        if (sj > m) m = sj;
    }
    for (int64_t d = 0; d < head_dim; ++d) out[d] = 0.0;
    if (m == -INFINITY) return; /* fully masked row (or no keys): output zero */
    double l = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        double p = exp(s[j] - m); /* exp(-inf) = 0 for masked keys */
        s[j] = p;
        l += p;
    }
    for (int64_t j = 0; j < n_keys; ++j) {
        if (s[j] == 0.0) continue;
        for (int64_t d = 0; d < head_dim; ++d) out[d] += s[j] * load_elem(v.base, v.dtype, v_off[j] + d);
    }
    for (int64_t d = 0; d < head_dim; ++d) out[d] /= l;
}

/* ---------------------------------------------------------------------------
 * O1: batched, strided, masked grouped-query attention.
 * For batch b, query row i < rows, head h < n_heads, kv head kh = h / g with
 * g = n_heads / n_kv_heads ([prefill]: one KV head per n_heads/n_kv_heads
 * query heads; consecutive query heads share), keys j < kv_len.
 * Strides are in elements, as on the [prefill] page.  The mask (optional) is
 * indexed mask[b*m_bs + h*m_hs + i*m_rs + j]; m_hs = 0 shares one mask across
 * heads as the [prefill] page does.  Output is double.
 * ------------------------------------------------------------------------- */
void oracle_attention(int64_t batch, int64_t rows, int64_t kv_len, int64_t n_heads,
                      int64_t n_kv_heads, int64_t head_dim, double scale,
                      const void *q, int q_dtype, int64_t q_bs, int64_t q_rs, int64_t q_hs,
                      const void *k, int k_dtype, int64_t k_bs, int64_t k_rs, int64_t k_hs,
                      const void *v, int v_dtype, int64_t v_bs, int64_t v_rs, int64_t v_hs,
                      const void *mask, int m_dtype, int64_t m_bs, int64_t m_hs, int64_t m_rs,
                      double *o, int64_t o_bs, int64_t o_rs, int64_t o_hs) {
    int64_t g = n_heads / n_kv_heads;
    int64_t total = batch * rows * n_heads;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(kv_len > 0 ? kv_len : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)head_dim);
        double *orow = (double *)malloc(sizeof(double) * (size_t)head_dim);
        int64_t *k_off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(kv_len > 0 ? kv_len : 1));
        int64_t *v_off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(kv_len > 0 ? kv_len : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < total; ++t) {
            int64_t b = t / (rows * n_heads);
            int64_t i = (t / n_heads) % rows;
            int64_t h = t % n_heads;
            int64_t kh = h / g;
            for (int64_t d = 0; d < head_dim; ++d)
                qrow[d] = load_elem(q, q_dtype, b * q_bs + i * q_rs + h * q_hs + d);
            for (int64_t j = 0; j < kv_len; ++j) {
                k_off[j] = b * k_bs + j * k_rs + kh * k_hs;
                v_off[j] = b * v_bs + j * v_rs + kh * v_hs;
            }
            elem_ref kr = {k, k_dtype}, vr = {v, v_dtype}, mr = {mask, m_dtype};
            attend_row(kv_len, head_dim, scale, qrow, kr, k_off, vr, v_off, mr,
                       b * m_bs + h * m_hs + i * m_rs, 1, mask != NULL, s, orow);
            for (int64_t d = 0; d < head_dim; ++d) o[b * o_bs + i * o_rs + h * o_hs + d] = orow[d];
        }
        free(s);
        free(qrow);
        free(orow);
        free(k_off);
        free(v_off);
    }
}

/* ---------------------------------------------------------------------------
 * O2: single-query attention over a paged KV cache ([paged]: pages of fixed
 * size, a per-sequence page table, the context extent is the position of the
 * new token plus the tokens written, so the query sees its own key).
 * Token t of sequence b lives in page page_table[b*max_pages + t/page_size],
 * slot t % page_size; its K row (kv head kh) starts at
 *   page*page_stride + slot*token_stride + kh*head_stride
 * (elements) in k_pool, and likewise in v_pool.  No mask.
 * Q and O are [batch, n_heads, head_dim] with strides q_bs/q_hs, o_bs/o_hs.
 * ------------------------------------------------------------------------- */
void oracle_paged_decode(int64_t batch, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
                         int64_t page_size, int64_t max_pages, double scale,
                         const void *q, int q_dtype, int64_t q_bs, int64_t q_hs,
                         const void *k_pool, const void *v_pool, int kv_dtype,
                         int64_t page_stride, int64_t token_stride, int64_t head_stride,
                         const int32_t *page_table, const int32_t *context_lens,
                         double *o, int64_t o_bs, int64_t o_hs) {
    int64_t g = n_heads / n_kv_heads;
    int64_t total = batch * n_heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < total; ++t) {
        int64_t b = t / n_heads;
        int64_t h = t % n_heads;
        int64_t kh = h / g;
        int64_t ctx = context_lens[b];
        if (ctx < 0) ctx = 0;
        double *s = (double *)malloc(sizeof(double) * (size_t)(ctx > 0 ? ctx : 1));
        int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(ctx > 0 ? ctx : 1));
        double *qrow = (double *)malloc(sizeof(double) * (size_t)head_dim);
        double *orow = (double *)malloc(sizeof(double) * (size_t)head_dim);
        for (int64_t d = 0; d < head_dim; ++d) qrow[d] = load_elem(q, q_dtype, b * q_bs + h * q_hs + d);
        for (int64_t tok = 0; tok < ctx; ++tok) {
            int64_t page = page_table[b * max_pages + tok / page_size];
            int64_t slot = tok % page_size;
            off[tok] = page * page_stride + slot * token_stride + kh * head_stride;
        }
        elem_ref kr = {k_pool, kv_dtype}, vr = {v_pool, kv_dtype}, none = {NULL, ORC_F64};
        attend_row(ctx, head_dim, scale, qrow, kr, off, vr, off, none, 0, 0, 0, s, orow);
        for (int64_t d = 0; d < head_dim; ++d) o[b * o_bs + h * o_hs + d] = orow[d];
        free(s);
        free(off);
        free(qrow);
        free(orow);
    }
}

/* ---------------------------------------------------------------------------
 * DFlash2 ring steps ([pack]).  Geometry (lanes b, q_heads h, kv_heads hk,
 * head_dim d, rows r, window w, packed_len k = w - 1 + r, max_commit c) as in
 * DFlash2AttentionPackParams.  Buffer shapes as the page's dispatch functions
 * require them, all contiguous:
 *   ring K/V      bf16 [b, hk, w, d]      current Q f32 [b, r, h, d]
 *   current K/V   f32  [b, r, hk, d]      packed Q bf16 [b, h, r, d]
 *   packed K/V    bf16 [b, hk, k, d]      mask      bf16 [b, h, r, k]
 *   new K/V       f32  [b, c, hk, d]      lengths, positions, counts u32 [b]
 * ------------------------------------------------------------------------- */
#define BF16_ZERO 0x0000u
#define BF16_NEG_INF 0xff80u

static int64_t ring_mod(int64_t x, int64_t w) {
    int64_t r = x % w;
    return r < 0 ? r + w : r;
}

/* O3: pack.  Packed position p < r holds drafted row p (current K/V, in
 * order); packed position p = r + j holds the j-th newest cached row, ring
 * slot (wp - 1 - j) mod w, while j < L; slots j >= L hold zero (a convention:
 * those positions are always masked, and the pages do not show what the
 * kernel writes there).  Worked example on the page: ring [1,2,3,4], wp = 1,
 * L = 3, drafted keys 20, 21 pack to [20, 21, 1, 4, 3]. */
void oracle_dflash_pack(int64_t lanes, int64_t q_heads, int64_t kv_heads, int64_t head_dim,
                        int64_t rows, int64_t window,
                        const uint16_t *ring_k, const uint16_t *ring_v,
                        const float *cur_q, const float *cur_k, const float *cur_v,
                        const uint32_t *cache_lengths, const uint32_t *write_positions,
                        uint16_t *packed_q, uint16_t *packed_k, uint16_t *packed_v) {
    int64_t b_, h, kh, i, p, d;
    int64_t packed_len = window - 1 + rows;
    for (b_ = 0; b_ < lanes; ++b_) {
        for (h = 0; h < q_heads; ++h)
            for (i = 0; i < rows; ++i)
                for (d = 0; d < head_dim; ++d)
                    packed_q[((b_ * q_heads + h) * rows + i) * head_dim + d] =
                        oracle_bf16_from_f32(cur_q[((b_ * rows + i) * q_heads + h) * head_dim + d]);
        int64_t L = cache_lengths[b_];
        int64_t wp = write_positions[b_];
        for (kh = 0; kh < kv_heads; ++kh) {
            for (p = 0; p < packed_len; ++p) {
                uint16_t *dk = packed_k + ((b_ * kv_heads + kh) * packed_len + p) * head_dim;
                uint16_t *dv = packed_v + ((b_ * kv_heads + kh) * packed_len + p) * head_dim;
                if (p < rows) {
                    const float *sk = cur_k + ((b_ * rows + p) * kv_heads + kh) * head_dim;
                    const float *sv = cur_v + ((b_ * rows + p) * kv_heads + kh) * head_dim;
                    for (d = 0; d < head_dim; ++d) {
                        dk[d] = oracle_bf16_from_f32(sk[d]);
                        dv[d] = oracle_bf16_from_f32(sv[d]);
                    }
                } else {
                    int64_t j = p - rows;
                    if (j < L) {
                        int64_t slot = ring_mod(wp - 1 - j, window);
                        const uint16_t *sk = ring_k + ((b_ * kv_heads + kh) * window + slot) * head_dim;
                        const uint16_t *sv = ring_v + ((b_ * kv_heads + kh) * window + slot) * head_dim;
                        for (d = 0; d < head_dim; ++d) {
                            dk[d] = sk[d];
                            dv[d] = sv[d];
                        }
                    } else {
                        for (d = 0; d < head_dim; ++d) {
                            dk[d] = BF16_ZERO;
                            dv[d] = BF16_ZERO;
                        }
                    }
                }
            }
        }
    }
}

/* O4: mask.  Query row i sees every drafted position p < r (the page's
 * example has row 0 seeing packed position 1, a drafted row after it), and
 * cached position j = p - r while j < min(L, w - 1 - i): a window of w
 * tokens ending at the row's own position (the example masks only row 1's
 * oldest cached key).  Visible = bf16 0, hidden = bf16 -inf; identical for
 * every head. */
void oracle_dflash_mask(int64_t lanes, int64_t q_heads, int64_t rows, int64_t window,
                        const uint32_t *cache_lengths, uint16_t *mask) {
    int64_t packed_len = window - 1 + rows;
    for (int64_t b_ = 0; b_ < lanes; ++b_) {
        int64_t L = cache_lengths[b_];
        for (int64_t h = 0; h < q_heads; ++h)
            for (int64_t i = 0; i < rows; ++i) {
                int64_t reach = window - 1 - i;
                if (L < reach) reach = L;
                for (int64_t p = 0; p < packed_len; ++p) {
                    int visible = (p < rows) || (p - rows < reach);
                    mask[((b_ * q_heads + h) * rows + i) * packed_len + p] =
                        (uint16_t)(visible ? BF16_ZERO : BF16_NEG_INF);
                }
            }
    }
}

/* O5: commit.  Row c < min(count, max_commit) of the new K/V goes, converted
 * to bf16, into ring slot (wp + c) mod w; every other ring element is left
 * alone.  The page's example commits 2 rows at wp = 1 into slots 1 and 2.
 * The kernel neither reads nor advances L / wp (the caller does). */
void oracle_dflash_commit(int64_t lanes, int64_t kv_heads, int64_t head_dim, int64_t window,
                          int64_t max_commit, const float *new_k, const float *new_v,
                          const uint32_t *commit_counts, const uint32_t *write_positions,
                          uint16_t *ring_k, uint16_t *ring_v) {
    for (int64_t b_ = 0; b_ < lanes; ++b_) {
        int64_t n = commit_counts[b_];
        if (n > max_commit) n = max_commit;
        int64_t wp = write_positions[b_];
        for (int64_t c = 0; c < n; ++c) {
            int64_t slot = ring_mod(wp + c, window);
            for (int64_t kh = 0; kh < kv_heads; ++kh) {
                const float *sk = new_k + ((b_ * max_commit + c) * kv_heads + kh) * head_dim;
                const float *sv = new_v + ((b_ * max_commit + c) * kv_heads + kh) * head_dim;
                uint16_t *dk = ring_k + ((b_ * kv_heads + kh) * window + slot) * head_dim;
                uint16_t *dv = ring_v + ((b_ * kv_heads + kh) * window + slot) * head_dim;
                for (int64_t d = 0; d < head_dim; ++d) {
                    dk[d] = oracle_bf16_from_f32(sk[d]);
                    dv[d] = oracle_bf16_from_f32(sv[d]);
                }
            }
        }
    }
}

/* Mask-rows step ([pack], the fourth kernel and its anchor test): rows
 * 1..r-1 of each lane's f32 draft input [lanes*r, hidden] are overwritten by
 * the bf16 mask embedding [hidden], widened to f32; row 0 (the anchor) is
 * kept.  Example on the page: [[7,8,9],[0,0,0]] with embedding [2,3,4]
 * becomes [[7,8,9],[2,3,4]]. */
void oracle_dflash_mask_rows(int64_t lanes, int64_t rows, int64_t hidden,
                             const uint16_t *mask_embedding, float *draft_input) {
    for (int64_t b_ = 0; b_ < lanes; ++b_)
        for (int64_t i = 1; i < rows; ++i)
            for (int64_t x = 0; x < hidden; ++x)
                draft_input[(b_ * rows + i) * hidden + x] = (float)oracle_bf16_to_f64(mask_embedding[x]);
}
