// api.hip -- the extern "C" entry points of libattn.so: argument validation,
// workspace sizing and kernel launch.  Every host-checkable rule is checked
// before anything is enqueued, as the dispatch functions on the
// mlx-native 0.18.0 flash_attn_prefill_tensor.rs and 0.21.1
// dflash2_attention_pack.rs pages validate before encoding; a violation
// returns ATTN_EINVAL with a message that includes the parameters.
#include <cmath>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "internal.h"

#ifndef ATTN_SOURCE_SHA256
#define ATTN_SOURCE_SHA256 "unknown"
#endif

namespace {

thread_local std::string g_last_error;

int fail(const char *fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return ATTN_EINVAL;
}

int hip_status(hipError_t err, const char *what) {
    if (err == hipSuccess) return ATTN_OK;
    char buf[512];
    snprintf(buf, sizeof buf, "%s: HIP error %d (%s)", what, (int)err, hipGetErrorString(err));
    g_last_error = buf;
    return ATTN_EHIP;
}

bool aligned(const void *ptr, uintptr_t n) { return ((uintptr_t)ptr % n) == 0; }

// Largest element index + 1 addressed by (count_i - 1) * stride_i summed, plus width.
// Returns false on overflow.
bool extent(int64_t *out, std::initializer_list<std::pair<int64_t, int64_t>> dims, int64_t width) {
    int64_t total = width;
    for (const auto &d : dims) {
        if (d.first <= 0) continue;
        int64_t term;
        if (__builtin_mul_overflow(d.first - 1, d.second, &term)) return false;
        if (__builtin_add_overflow(total, term, &total)) return false;
    }
    *out = total;
    return true;
}

const int kMaxGridYZ = 65535;

std::string prefill_dump(const attn_prefill_params *p) {
    char buf[768];
    snprintf(buf, sizeof buf,
             "{batch=%d rows=%d kv_len=%d n_heads=%d n_kv_heads=%d head_dim=%d q_dtype=%d kv_dtype=%d "
             "mask_dtype=%d scale=%g q=(%lld,%lld,%lld) k=(%lld,%lld,%lld) v=(%lld,%lld,%lld) "
             "m=(%lld,%lld,%lld) o=(%lld,%lld,%lld) caps=(%lld,%lld,%lld,%lld,%lld)}",
             p->batch, p->rows, p->kv_len, p->n_heads, p->n_kv_heads, p->head_dim, p->q_dtype, p->kv_dtype,
             p->mask_dtype, (double)p->scale, (long long)p->q_bs, (long long)p->q_rs, (long long)p->q_hs,
             (long long)p->k_bs, (long long)p->k_rs, (long long)p->k_hs, (long long)p->v_bs, (long long)p->v_rs,
             (long long)p->v_hs, (long long)p->m_bs, (long long)p->m_hs, (long long)p->m_rs, (long long)p->o_bs,
             (long long)p->o_rs, (long long)p->o_hs, (long long)p->q_cap, (long long)p->k_cap,
             (long long)p->v_cap, (long long)p->m_cap, (long long)p->o_cap);
    return buf;
}

int check_prefill(const attn_prefill_params *p, attn::PrefillPlan *plan) {
    if (!p) return fail("attn_prefill: params is NULL");
    const std::string dump = prefill_dump(p);
    const char *d = dump.c_str();
    if (p->batch <= 0 || p->rows <= 0 || p->kv_len <= 0 || p->n_heads <= 0 || p->n_kv_heads <= 0)
        return fail("attn_prefill: empty shape %s", d);
    if (p->n_heads % p->n_kv_heads != 0)
        return fail("attn_prefill: n_heads %d is not a multiple of n_kv_heads %d", p->n_heads, p->n_kv_heads);
    if (p->head_dim != 128 && p->head_dim != 256 && p->head_dim != 512)
        return fail("attn_prefill: unsupported head_dim %d (128, 256 or 512) %s", p->head_dim, d);
    if (p->q_dtype != ATTN_F32 && p->q_dtype != ATTN_BF16)
        return fail("attn_prefill: q_dtype must be F32 or BF16 %s", d);
    if (p->kv_dtype != ATTN_F16 && p->kv_dtype != ATTN_BF16)
        return fail("attn_prefill: kv_dtype must be F16 or BF16 %s", d);
    if (p->mask_dtype != ATTN_NONE && p->mask_dtype != ATTN_F16 && p->mask_dtype != ATTN_BF16)
        return fail("attn_prefill: mask_dtype must be NONE, F16 or BF16 %s", d);
    const int64_t strides[] = {p->q_bs, p->q_rs, p->q_hs, p->k_bs, p->k_rs, p->k_hs, p->v_bs, p->v_rs,
                               p->v_hs, p->m_bs, p->m_hs, p->m_rs, p->o_bs, p->o_rs, p->o_hs};
    for (int64_t s : strides)
        if (s < 0) return fail("attn_prefill: negative stride %s", d);
    const int qa = p->q_dtype == ATTN_F32 ? 4 : 8;
    if (p->q_bs % qa || p->q_rs % qa || p->q_hs % qa)
        return fail("attn_prefill: Q strides must be multiples of %d (128-bit loads) %s", qa, d);
    if (p->k_bs % 8 || p->k_rs % 8 || p->k_hs % 8 || p->v_bs % 8 || p->v_rs % 8 || p->v_hs % 8)
        return fail("attn_prefill: K/V strides must be multiples of 8 (128-bit loads) %s", d);
    if (p->o_bs % 4 || p->o_rs % 4 || p->o_hs % 4)
        return fail("attn_prefill: O strides must be multiples of 4 %s", d);
    int64_t need;
    if (!extent(&need, {{p->batch, p->q_bs}, {p->rows, p->q_rs}, {p->n_heads, p->q_hs}}, p->head_dim) ||
        need > p->q_cap)
        return fail("attn_prefill: q holds %lld elements, the strides need more %s", (long long)p->q_cap, d);
    if (!extent(&need, {{p->batch, p->k_bs}, {p->kv_len, p->k_rs}, {p->n_kv_heads, p->k_hs}}, p->head_dim) ||
        need > p->k_cap)
        return fail("attn_prefill: k holds %lld elements, the strides need more %s", (long long)p->k_cap, d);
    if (!extent(&need, {{p->batch, p->v_bs}, {p->kv_len, p->v_rs}, {p->n_kv_heads, p->v_hs}}, p->head_dim) ||
        need > p->v_cap)
        return fail("attn_prefill: v holds %lld elements, the strides need more %s", (long long)p->v_cap, d);
    if (p->mask_dtype != ATTN_NONE &&
        (!extent(&need, {{p->batch, p->m_bs}, {p->n_heads, p->m_hs}, {p->rows, p->m_rs}}, p->kv_len) ||
         need > p->m_cap))
        return fail("attn_prefill: mask holds %lld elements, the strides need more %s", (long long)p->m_cap, d);
    if (!extent(&need, {{p->batch, p->o_bs}, {p->rows, p->o_rs}, {p->n_heads, p->o_hs}}, p->head_dim) ||
        need > p->o_cap)
        return fail("attn_prefill: out holds %lld elements, the strides need more %s", (long long)p->o_cap, d);
    if (attn::plan_prefill(p, plan) != ATTN_OK) return fail("attn_prefill: no launch shape fits %s", d);
    const int64_t blk_heads = (p->mask_dtype != ATTN_NONE && p->m_hs != 0) ? plan->head_groups : 1;
    if (plan->head_groups > kMaxGridYZ || (int64_t)p->batch * plan->splits > kMaxGridYZ ||
        plan->row_blocks > kMaxGridYZ || (int64_t)p->batch * blk_heads > kMaxGridYZ)
        return fail("attn_prefill: grid too large %s", d);
    return ATTN_OK;
}

std::string decode_dump(const attn_decode_params *p) {
    char buf[512];
    snprintf(buf, sizeof buf,
             "{batch=%d n_heads=%d n_kv_heads=%d head_dim=%d page_size=%d max_pages_per_seq=%d num_pages=%d "
             "max_context=%d kv_dtype=%d scale=%g q=(%lld,%lld) o=(%lld,%lld) kv=(%lld,%lld,%lld) "
             "caps=(%lld,%lld,%lld)}",
             p->batch, p->n_heads, p->n_kv_heads, p->head_dim, p->page_size, p->max_pages_per_seq, p->num_pages,
             p->max_context, p->kv_dtype, (double)p->scale, (long long)p->q_bs, (long long)p->q_hs,
             (long long)p->o_bs, (long long)p->o_hs, (long long)p->kv_page_stride, (long long)p->kv_token_stride,
             (long long)p->kv_head_stride, (long long)p->q_cap, (long long)p->kv_cap, (long long)p->o_cap);
    return buf;
}

int check_decode(const attn_decode_params *p, attn::DecodePlan *plan) {
    if (!p) return fail("attn_paged_decode: params is NULL");
    const std::string dump = decode_dump(p);
    const char *d = dump.c_str();
    if (p->batch <= 0 || p->n_heads <= 0 || p->n_kv_heads <= 0 || p->page_size <= 0 || p->max_pages_per_seq <= 0 ||
        p->num_pages <= 0 || p->max_context < 0)
        return fail("attn_paged_decode: empty or negative shape %s", d);
    if (p->n_heads % p->n_kv_heads != 0)
        return fail("attn_paged_decode: n_heads %d is not a multiple of n_kv_heads %d", p->n_heads, p->n_kv_heads);
    if (p->head_dim != 128 && p->head_dim != 256)
        return fail("attn_paged_decode: unsupported head_dim %d (128 or 256) %s", p->head_dim, d);
    if (p->kv_dtype != ATTN_F16 && p->kv_dtype != ATTN_BF16)
        return fail("attn_paged_decode: kv_dtype must be F16 or BF16 %s", d);
    if (p->q_bs < 0 || p->q_hs < 0 || p->o_bs < 0 || p->o_hs < 0 || p->kv_page_stride < 0 ||
        p->kv_token_stride < 0 || p->kv_head_stride < 0)
        return fail("attn_paged_decode: negative stride %s", d);
    if (p->q_bs % 4 || p->q_hs % 4 || p->o_bs % 4 || p->o_hs % 4)
        return fail("attn_paged_decode: Q/O strides must be multiples of 4 %s", d);
    if (p->kv_page_stride % 8 || p->kv_token_stride % 8 || p->kv_head_stride % 8)
        return fail("attn_paged_decode: KV strides must be multiples of 8 (128-bit loads) %s", d);
    int64_t need;
    if (!extent(&need, {{p->batch, p->q_bs}, {p->n_heads, p->q_hs}}, p->head_dim) || need > p->q_cap)
        return fail("attn_paged_decode: q holds %lld elements, the strides need more %s", (long long)p->q_cap, d);
    if (!extent(&need, {{p->batch, p->o_bs}, {p->n_heads, p->o_hs}}, p->head_dim) || need > p->o_cap)
        return fail("attn_paged_decode: out holds %lld elements, the strides need more %s", (long long)p->o_cap, d);
    if (!extent(&need, {{p->num_pages, p->kv_page_stride}, {p->page_size, p->kv_token_stride},
                        {p->n_kv_heads, p->kv_head_stride}},
                p->head_dim) ||
        need > p->kv_cap)
        return fail("attn_paged_decode: KV pools hold %lld elements, the strides need more %s", (long long)p->kv_cap,
                    d);
    attn::plan_decode(p, plan);
    if (plan->grid > (1ll << 31) - 1 || (int64_t)p->batch * p->n_heads / 4 + 1 > (1ll << 31) - 1)
        return fail("attn_paged_decode: grid too large %s", d);
    return ATTN_OK;
}

std::string paged_prefill_dump(const attn_paged_prefill_params *p) {
    char buf[640];
    snprintf(buf, sizeof buf,
             "{batch=%d n_heads=%d n_kv_heads=%d head_dim=%d page_size=%d max_pages_per_seq=%d num_pages=%d "
             "max_context=%d max_tokens=%d kv_dtype=%d scale=%g q=(%lld,%lld,%lld) o=(%lld,%lld,%lld) "
             "kv=(%lld,%lld,%lld) caps=(%lld,%lld,%lld)}",
             p->batch, p->n_heads, p->n_kv_heads, p->head_dim, p->page_size, p->max_pages_per_seq, p->num_pages,
             p->max_context, p->max_tokens, p->kv_dtype, (double)p->scale, (long long)p->q_bs, (long long)p->q_ts,
             (long long)p->q_hs, (long long)p->o_bs, (long long)p->o_ts, (long long)p->o_hs,
             (long long)p->kv_page_stride, (long long)p->kv_token_stride, (long long)p->kv_head_stride,
             (long long)p->q_cap, (long long)p->kv_cap, (long long)p->o_cap);
    return buf;
}

int check_paged_prefill(const attn_paged_prefill_params *p, attn::MultiPlan *plan, const char *who) {
    if (!p) return fail("%s: params is NULL", who);
    const std::string dump = paged_prefill_dump(p);
    const char *d = dump.c_str();
    if (p->batch <= 0 || p->n_heads <= 0 || p->n_kv_heads <= 0 || p->page_size <= 0 || p->max_pages_per_seq <= 0 ||
        p->num_pages <= 0 || p->max_context < 0)
        return fail("%s: empty or negative shape %s", who, d);
    if (p->max_tokens < 1 || p->max_tokens > attn::kMultiMaxTokens)
        return fail("%s: max_tokens %d outside [1, %d] %s", who, p->max_tokens, attn::kMultiMaxTokens, d);
    if (p->n_heads % p->n_kv_heads != 0)
        return fail("%s: n_heads %d is not a multiple of n_kv_heads %d", who, p->n_heads, p->n_kv_heads);
    if (p->head_dim != 128 && p->head_dim != 256)
        return fail("%s: unsupported head_dim %d (128 or 256) %s", who, p->head_dim, d);
    if (p->kv_dtype != ATTN_F16 && p->kv_dtype != ATTN_BF16) return fail("%s: kv_dtype must be F16 or BF16 %s", who, d);
    if (!std::isfinite(p->scale)) return fail("%s: scale must be finite %s", who, d);
    if (p->q_bs < 0 || p->q_ts < 0 || p->q_hs < 0 || p->o_bs < 0 || p->o_ts < 0 || p->o_hs < 0 ||
        p->kv_page_stride < 0 || p->kv_token_stride < 0 || p->kv_head_stride < 0)
        return fail("%s: negative stride %s", who, d);
    if (p->q_bs % 4 || p->q_ts % 4 || p->q_hs % 4 || p->o_bs % 4 || p->o_ts % 4 || p->o_hs % 4)
        return fail("%s: Q/O strides must be multiples of 4 %s", who, d);
    if (p->kv_page_stride % 8 || p->kv_token_stride % 8 || p->kv_head_stride % 8)
        return fail("%s: KV strides must be multiples of 8 (128-bit loads) %s", who, d);
    int64_t need;
    if (!extent(&need, {{p->batch, p->q_bs}, {p->max_tokens, p->q_ts}, {p->n_heads, p->q_hs}}, p->head_dim) ||
        need > p->q_cap)
        return fail("%s: q holds %lld elements, the strides need more %s", who, (long long)p->q_cap, d);
    if (!extent(&need, {{p->batch, p->o_bs}, {p->max_tokens, p->o_ts}, {p->n_heads, p->o_hs}}, p->head_dim) ||
        need > p->o_cap)
        return fail("%s: out holds %lld elements, the strides need more %s", who, (long long)p->o_cap, d);
    if (!extent(&need, {{p->num_pages, p->kv_page_stride}, {p->page_size, p->kv_token_stride},
                        {p->n_kv_heads, p->kv_head_stride}},
                p->head_dim) ||
        need > p->kv_cap)
        return fail("%s: KV pools hold %lld elements, the strides need more %s", who, (long long)p->kv_cap, d);
    attn::plan_paged_prefill(p, plan);
    if (plan->grid > (1ll << 31) - 1 || (int64_t)p->batch * p->max_tokens * p->n_heads / 4 + 1 > (1ll << 31) - 1)
        return fail("%s: grid too large %s", who, d);
    return ATTN_OK;
}

int check_prepare(const attn_paged_prepare_params *p) {
    if (!p) return fail("attn_paged_prepare: params is NULL");
    char buf[512];
    snprintf(buf, sizeof buf,
             "{batch=%d n_heads=%d n_kv_heads=%d head_dim=%d max_tokens=%d rope_dim=%d interleaved=%d qk_norm=%d "
             "page_size=%d max_pages_per_seq=%d num_pages=%d max_context=%d kv_dtype=%d eps=%g theta=%g}",
             p->batch, p->n_heads, p->n_kv_heads, p->head_dim, p->max_tokens, p->rope_dim, p->rope_interleaved,
             p->qk_norm, p->page_size, p->max_pages_per_seq, p->num_pages, p->max_context, p->kv_dtype,
             (double)p->epsilon, (double)p->rope_theta);
    const char *d = buf;
    if (p->batch <= 0 || p->n_heads <= 0 || p->n_kv_heads <= 0 || p->max_tokens <= 0 || p->page_size <= 0 ||
        p->max_pages_per_seq <= 0 || p->num_pages <= 0 || p->max_context < 0)
        return fail("attn_paged_prepare: empty or negative shape %s", d);
    if (p->n_heads % p->n_kv_heads != 0)
        return fail("attn_paged_prepare: n_heads %d is not a multiple of n_kv_heads %d", p->n_heads, p->n_kv_heads);
    if (p->head_dim != 128 && p->head_dim != 256)
        return fail("attn_paged_prepare: unsupported head_dim %d (128 or 256) %s", p->head_dim, d);
    if (p->rope_dim <= 0 || p->rope_dim > p->head_dim || p->rope_dim % 2)
        return fail("attn_paged_prepare: rope_dim must be even and in (0, head_dim] %s", d);
    if (p->kv_dtype != ATTN_F16 && p->kv_dtype != ATTN_BF16)
        return fail("attn_paged_prepare: kv_dtype must be F16 or BF16 %s", d);
    if (!std::isfinite(p->epsilon) || p->epsilon < 0.f || !std::isfinite(p->rope_theta) || p->rope_theta <= 0.f)
        return fail("attn_paged_prepare: epsilon must be finite and >= 0, rope_theta finite and > 0 %s", d);
    const int64_t strides[] = {p->qr_bs, p->qr_ts, p->qr_hs, p->kr_bs, p->kr_ts, p->kr_hs, p->vr_bs, p->vr_ts,
                               p->vr_hs, p->qo_bs, p->qo_ts, p->qo_hs, p->qn_hs, p->kn_hs, p->kv_page_stride,
                               p->kv_token_stride, p->kv_head_stride};
    for (int64_t st : strides)
        if (st < 0) return fail("attn_paged_prepare: negative stride %s", d);
    // 16-byte row accesses: every f32 stride a multiple of 4 elements, the pools' of 4 (8 bytes)
    for (int64_t st : strides)
        if (st % 4) return fail("attn_paged_prepare: strides must be multiples of 4 elements %s", d);
    int64_t need;
    const struct {
        const char *name;
        int64_t bs, ts, hs, heads, cap;
    } rows[] = {{"q_raw", p->qr_bs, p->qr_ts, p->qr_hs, p->n_heads, p->qr_cap},
                {"k_raw", p->kr_bs, p->kr_ts, p->kr_hs, p->n_kv_heads, p->kr_cap},
                {"v_raw", p->vr_bs, p->vr_ts, p->vr_hs, p->n_kv_heads, p->vr_cap},
                {"q_out", p->qo_bs, p->qo_ts, p->qo_hs, p->n_heads, p->qo_cap}};
    for (const auto &r : rows)
        if (!extent(&need, {{p->batch, r.bs}, {p->max_tokens, r.ts}, {r.heads, r.hs}}, p->head_dim) || need > r.cap)
            return fail("attn_paged_prepare: %s holds %lld elements, the strides need more %s", r.name,
                        (long long)r.cap, d);
    if (p->qk_norm) {
        if (!extent(&need, {{p->n_heads, p->qn_hs}}, p->head_dim) || need > p->qn_cap ||
            !extent(&need, {{p->n_kv_heads, p->kn_hs}}, p->head_dim) || need > p->kn_cap)
            return fail("attn_paged_prepare: norm weights hold too few elements %s", d);
    }
    if (!extent(&need, {{p->num_pages, p->kv_page_stride}, {p->page_size, p->kv_token_stride},
                        {p->n_kv_heads, p->kv_head_stride}},
                p->head_dim) ||
        need > p->kv_cap)
        return fail("attn_paged_prepare: KV pools hold %lld elements, the strides need more %s", (long long)p->kv_cap,
                    d);
    const int64_t items = (int64_t)p->batch * p->max_tokens * (p->n_heads + 2 * p->n_kv_heads);
    if ((items + 3) / 4 > (1ll << 31) - 1) return fail("attn_paged_prepare: grid too large %s", d);
    return ATTN_OK;
}

std::string dflash_dump(const dflash_params *p) {
    char buf[256];
    snprintf(buf, sizeof buf,
             "DFlash2AttentionPackParams { lanes: %u, q_heads: %u, kv_heads: %u, head_dim: %u, rows: %u, "
             "window: %u, packed_len: %u, max_commit: %u }",
             p->lanes, p->q_heads, p->kv_heads, p->head_dim, p->rows, p->window, p->packed_len, p->max_commit);
    return buf;
}

int check_dflash(const dflash_params *p, const char *who) {
    if (!p) return fail("%s: params is NULL", who);
    const bool bad = p->lanes == 0 || p->lanes > 4 || p->q_heads == 0 || p->kv_heads == 0 ||
                     p->q_heads % p->kv_heads != 0 || !(p->head_dim == 128 || p->head_dim == 256) ||
                     p->rows < 2 || p->rows > 16 || p->window <= p->rows ||
                     (uint64_t)p->packed_len != (uint64_t)p->window - 1 + p->rows || p->max_commit == 0 ||
                     p->max_commit > p->rows;
    if (bad) return fail("%s: invalid DFlash2 attention geometry: %s", who, dflash_dump(p).c_str());
    return ATTN_OK;
}

int check_verify(const dflash_params *p, attn::VerifyPlan *plan, const char *who) {
    int st = check_dflash(p, who);
    if (st != ATTN_OK) return st;
    if (p->window > attn::kVerifyMaxWindow)
        return fail("%s: window %u exceeds %u %s", who, p->window, attn::kVerifyMaxWindow, dflash_dump(p).c_str());
    attn::plan_verify(p, plan);
    if ((int64_t)p->kv_heads * plan->qgroups > kMaxGridYZ)
        return fail("%s: grid too large %s", who, dflash_dump(p).c_str());
    return ATTN_OK;
}

struct Need {
    const char *label;
    const void *ptr;
    uint64_t elems_a, elems_b, elems_c, elems_d;  // shape (0 = absent dimension)
    uint64_t elem_bytes;
    uintptr_t align;
};

int check_buffers(const char *who, const Need *needs, int n, const uint64_t *bytes) {
    if (!bytes) return fail("%s: byte lengths array is NULL", who);
    for (int i = 0; i < n; ++i) {
        const Need &nd = needs[i];
        unsigned __int128 want = nd.elem_bytes;
        for (uint64_t dim : {nd.elems_a, nd.elems_b, nd.elems_c, nd.elems_d})
            if (dim) want *= dim;
        if (want >> 62) return fail("%s: %s byte count overflows", who, nd.label);
        if (!nd.ptr) return fail("%s: %s is NULL", who, nd.label);
        if (!aligned(nd.ptr, nd.align)) return fail("%s: %s must be %u-byte aligned", who, nd.label, (unsigned)nd.align);
        if (bytes[i] != (uint64_t)want)
            return fail("%s: %s must be %llu bytes [%llu, %llu, %llu, %llu], got %llu bytes", who, nd.label,
                        (unsigned long long)want, (unsigned long long)nd.elems_a, (unsigned long long)nd.elems_b,
                        (unsigned long long)nd.elems_c, (unsigned long long)nd.elems_d,
                        (unsigned long long)bytes[i]);
    }
    return ATTN_OK;
}

}  // namespace

extern "C" {

const char *attn_last_error(void) { return g_last_error.c_str(); }

const char *attn_source_sha256(void) { return ATTN_SOURCE_SHA256; }

uint32_t attn_kv_pad(uint32_t kv_len) { return (kv_len + ATTN_KV_TILE - 1) / ATTN_KV_TILE * ATTN_KV_TILE; }

int attn_prefill_workspace_bytes(const attn_prefill_params *p, size_t *bytes) {
    attn::PrefillPlan plan;
    int st = check_prefill(p, &plan);
    if (st != ATTN_OK) return st;
    if (!bytes) return fail("attn_prefill_workspace_bytes: bytes is NULL");
    *bytes = plan.workspace_bytes;
    return ATTN_OK;
}

int attn_prefill(const attn_prefill_params *p, const void *q, const void *k, const void *v, const void *mask,
                 float *o, void *ws, size_t ws_bytes, void *stream) {
    attn::PrefillPlan plan;
    int st = check_prefill(p, &plan);
    if (st != ATTN_OK) return st;
    if (!q || !k || !v || !o) return fail("attn_prefill: q, k, v and out must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail("attn_prefill: q, k, v and out must be 16-byte aligned");
    if (p->mask_dtype != ATTN_NONE && (!mask || !aligned(mask, 2)))
        return fail("attn_prefill: mask must be a non-NULL, 2-byte aligned pointer when mask_dtype is set");
    if (plan.workspace_bytes > 0 && (!ws || ws_bytes < plan.workspace_bytes || !aligned(ws, 16)))
        return fail("attn_prefill: workspace needs %zu bytes (16-byte aligned), got %zu", plan.workspace_bytes,
                    ws ? ws_bytes : (size_t)0);
    return hip_status(attn::launch_prefill(p, &plan, q, k, v, mask, o, ws, (hipStream_t)stream), "attn_prefill");
}

int attn_paged_decode_workspace_bytes(const attn_decode_params *p, size_t *bytes) {
    attn::DecodePlan plan;
    int st = check_decode(p, &plan);
    if (st != ATTN_OK) return st;
    if (!bytes) return fail("attn_paged_decode_workspace_bytes: bytes is NULL");
    *bytes = plan.workspace_bytes;
    return ATTN_OK;
}

int attn_paged_decode(const attn_decode_params *p, const float *q, const void *k_pool, const void *v_pool,
                      const int32_t *page_table, const int32_t *context_lens, float *o, void *ws, size_t ws_bytes,
                      void *stream) {
    attn::DecodePlan plan;
    int st = check_decode(p, &plan);
    if (st != ATTN_OK) return st;
    if (!q || !k_pool || !v_pool || !page_table || !context_lens || !o)
        return fail("attn_paged_decode: every buffer must be non-NULL");
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
        !aligned(page_table, 4) || !aligned(context_lens, 4))
        return fail("attn_paged_decode: q, pools and out must be 16-byte aligned, tables 4-byte aligned");
    if (!ws || ws_bytes < plan.workspace_bytes || !aligned(ws, 16))
        return fail("attn_paged_decode: workspace needs %zu bytes (16-byte aligned), got %zu", plan.workspace_bytes,
                    ws ? ws_bytes : (size_t)0);
    return hip_status(attn::launch_paged_decode(p, &plan, q, k_pool, v_pool, page_table, context_lens, o, ws,
                                                (hipStream_t)stream),
                      "attn_paged_decode");
}

int attn_paged_decode_noalloc(const attn_decode_params *p, const float *q, const void *k_pool, const void *v_pool,
                              const int32_t *page_table, const int32_t *context_lens, float *o, void *stream) {
    attn::DecodePlan plan;
    int st = check_decode(p, &plan);
    if (st != ATTN_OK) return st;
    if (!q || !k_pool || !v_pool || !page_table || !context_lens || !o)
        return fail("attn_paged_decode_noalloc: every buffer must be non-NULL");
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
        !aligned(page_table, 4) || !aligned(context_lens, 4))
        return fail("attn_paged_decode_noalloc: q, pools and out must be 16-byte aligned, tables 4-byte aligned");
    if (plan.workspace_bytes > ATTN_DECODE_SCRATCH_BYTES)
        return fail("attn_paged_decode_noalloc: the call needs %zu bytes of scratch, more than the %zu the library "
                    "holds; use attn_paged_decode with a workspace",
                    plan.workspace_bytes, (size_t)ATTN_DECODE_SCRATCH_BYTES);
    void *scratch = nullptr;
    if (attn::decode_scratch(&scratch) != ATTN_OK) {
        g_last_error = "attn_paged_decode_noalloc: no scratch address for the current device";
        return ATTN_EHIP;
    }
    return hip_status(attn::launch_paged_decode(p, &plan, q, k_pool, v_pool, page_table, context_lens, o, scratch,
                                                (hipStream_t)stream),
                      "attn_paged_decode_noalloc");
}

int attn_paged_prefill_workspace_bytes(const attn_paged_prefill_params *p, size_t *bytes) {
    attn::MultiPlan plan;
    int st = check_paged_prefill(p, &plan, "attn_paged_prefill_workspace_bytes");
    if (st != ATTN_OK) return st;
    if (!bytes) return fail("attn_paged_prefill_workspace_bytes: bytes is NULL");
    *bytes = plan.workspace_bytes;
    return ATTN_OK;
}

int attn_paged_prefill(const attn_paged_prefill_params *p, const float *q, const void *k_pool, const void *v_pool,
                       const int32_t *page_table, const int32_t *query_lens, const int32_t *position_starts,
                       float *o, void *ws, size_t ws_bytes, void *stream) {
    attn::MultiPlan plan;
    int st = check_paged_prefill(p, &plan, "attn_paged_prefill");
    if (st != ATTN_OK) return st;
    if (!q || !k_pool || !v_pool || !page_table || !query_lens || !position_starts || !o)
        return fail("attn_paged_prefill: every buffer must be non-NULL");
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
        !aligned(page_table, 4) || !aligned(query_lens, 4) || !aligned(position_starts, 4))
        return fail("attn_paged_prefill: q, pools and out must be 16-byte aligned, tables 4-byte aligned");
    if (!ws || ws_bytes < plan.workspace_bytes || !aligned(ws, 16))
        return fail("attn_paged_prefill: workspace needs %zu bytes (16-byte aligned), got %zu", plan.workspace_bytes,
                    ws ? ws_bytes : (size_t)0);
    return hip_status(attn::launch_paged_prefill(p, &plan, q, k_pool, v_pool, page_table, query_lens, position_starts,
                                                 o, ws, (hipStream_t)stream),
                      "attn_paged_prefill");
}

int attn_paged_prepare(const attn_paged_prepare_params *p, const float *q_raw, const float *k_raw, const float *v_raw,
                       const float *q_norm, const float *k_norm, const int32_t *page_table, const int32_t *query_lens,
                       const int32_t *position_starts, float *q_out, void *k_pool, void *v_pool, void *stream) {
    int st = check_prepare(p);
    if (st != ATTN_OK) return st;
    if (!q_raw || !k_raw || !v_raw || !page_table || !query_lens || !position_starts || !q_out || !k_pool || !v_pool)
        return fail("attn_paged_prepare: every buffer must be non-NULL");
    if (p->qk_norm && (!q_norm || !k_norm)) return fail("attn_paged_prepare: qk_norm needs both norm weight buffers");
    if (!aligned(q_raw, 16) || !aligned(k_raw, 16) || !aligned(v_raw, 16) || !aligned(q_out, 16) ||
        !aligned(k_pool, 8) || !aligned(v_pool, 8) || !aligned(page_table, 4) || !aligned(query_lens, 4) ||
        !aligned(position_starts, 4) || (p->qk_norm && (!aligned(q_norm, 16) || !aligned(k_norm, 16))))
        return fail("attn_paged_prepare: f32 buffers must be 16-byte aligned, the pools 8-byte, the tables 4-byte");
    return hip_status(attn::launch_paged_prepare(p, q_raw, k_raw, v_raw, q_norm, k_norm, page_table, query_lens,
                                                 position_starts, q_out, k_pool, v_pool, (hipStream_t)stream),
                      "attn_paged_prepare");
}

int dflash_validate(const dflash_params *p) { return check_dflash(p, "dflash_validate"); }

int dflash_pack(const dflash_params *p, const uint16_t *ring_k, const uint16_t *ring_v, const float *cur_q,
                const float *cur_k, const float *cur_v, const uint32_t *cache_lengths,
                const uint32_t *write_positions, uint16_t *packed_q, uint16_t *packed_k, uint16_t *packed_v,
                const uint64_t *bytes, void *stream) {
    int st = check_dflash(p, "dflash_pack");
    if (st != ATTN_OK) return st;
    const uint64_t b = p->lanes, h = p->q_heads, hk = p->kv_heads, d = p->head_dim, r = p->rows, w = p->window,
                   k = p->packed_len;
    const Need needs[] = {
        {"ring keys", ring_k, b, hk, w, d, 2, 16},          {"ring values", ring_v, b, hk, w, d, 2, 16},
        {"current queries", cur_q, b, r, h, d, 4, 16},      {"current keys", cur_k, b, r, hk, d, 4, 16},
        {"current values", cur_v, b, r, hk, d, 4, 16},      {"cache lengths", cache_lengths, b, 0, 0, 0, 4, 4},
        {"write positions", write_positions, b, 0, 0, 0, 4, 4}, {"packed queries", packed_q, b, h, r, d, 2, 16},
        {"packed keys", packed_k, b, hk, k, d, 2, 16},      {"packed values", packed_v, b, hk, k, d, 2, 16},
    };
    st = check_buffers("dflash_pack", needs, 10, bytes);
    if (st != ATTN_OK) return st;
    return hip_status(attn::launch_dflash_pack(p, ring_k, ring_v, cur_q, cur_k, cur_v, cache_lengths,
                                               write_positions, packed_q, packed_k, packed_v, (hipStream_t)stream),
                      "dflash_pack");
}

int dflash_mask(const dflash_params *p, const uint32_t *cache_lengths, uint16_t *mask, const uint64_t *bytes,
                void *stream) {
    int st = check_dflash(p, "dflash_mask");
    if (st != ATTN_OK) return st;
    const Need needs[] = {
        {"cache lengths", cache_lengths, p->lanes, 0, 0, 0, 4, 4},
        {"mask", mask, p->lanes, p->q_heads, p->rows, p->packed_len, 2, 16},
    };
    st = check_buffers("dflash_mask", needs, 2, bytes);
    if (st != ATTN_OK) return st;
    return hip_status(attn::launch_dflash_mask(p, cache_lengths, mask, (hipStream_t)stream), "dflash_mask");
}

int dflash_commit(const dflash_params *p, const float *new_k, const float *new_v, const uint32_t *commit_counts,
                  const uint32_t *write_positions, uint16_t *ring_k, uint16_t *ring_v, const uint64_t *bytes,
                  void *stream) {
    int st = check_dflash(p, "dflash_commit");
    if (st != ATTN_OK) return st;
    const uint64_t b = p->lanes, hk = p->kv_heads, d = p->head_dim, w = p->window, c = p->max_commit;
    const Need needs[] = {
        {"new keys", new_k, b, c, hk, d, 4, 16},          {"new values", new_v, b, c, hk, d, 4, 16},
        {"commit counts", commit_counts, b, 0, 0, 0, 4, 4}, {"write positions", write_positions, b, 0, 0, 0, 4, 4},
        {"ring keys", ring_k, b, hk, w, d, 2, 16},        {"ring values", ring_v, b, hk, w, d, 2, 16},
    };
    st = check_buffers("dflash_commit", needs, 6, bytes);
    if (st != ATTN_OK) return st;
    return hip_status(attn::launch_dflash_commit(p, new_k, new_v, commit_counts, write_positions, ring_k, ring_v,
                                                 (hipStream_t)stream),
                      "dflash_commit");
}

int dflash_verify_workspace_bytes(const dflash_params *p, size_t *bytes) {
    attn::VerifyPlan plan;
    int st = check_verify(p, &plan, "dflash_verify_workspace_bytes");
    if (st != ATTN_OK) return st;
    if (!bytes) return fail("dflash_verify_workspace_bytes: bytes is NULL");
    *bytes = plan.workspace_bytes;
    return ATTN_OK;
}

int dflash_verify_attention(const dflash_params *p, float scale, const uint16_t *ring_k, const uint16_t *ring_v,
                            const float *cur_q, const float *cur_k, const float *cur_v,
                            const uint32_t *cache_lengths, const uint32_t *write_positions, float *out, void *ws,
                            size_t ws_bytes, const uint64_t *bytes, void *stream) {
    attn::VerifyPlan plan;
    int st = check_verify(p, &plan, "dflash_verify_attention");
    if (st != ATTN_OK) return st;
    if (!std::isfinite(scale)) return fail("dflash_verify_attention: scale must be finite, got %g", (double)scale);
    const uint64_t b = p->lanes, h = p->q_heads, hk = p->kv_heads, d = p->head_dim, r = p->rows, w = p->window;
    const Need needs[] = {
        {"ring keys", ring_k, b, hk, w, d, 2, 16},          {"ring values", ring_v, b, hk, w, d, 2, 16},
        {"current queries", cur_q, b, r, h, d, 4, 16},      {"current keys", cur_k, b, r, hk, d, 4, 16},
        {"current values", cur_v, b, r, hk, d, 4, 16},      {"cache lengths", cache_lengths, b, 0, 0, 0, 4, 4},
        {"write positions", write_positions, b, 0, 0, 0, 4, 4}, {"output", out, b, h, r, d, 4, 16},
    };
    st = check_buffers("dflash_verify_attention", needs, 8, bytes);
    if (st != ATTN_OK) return st;
    if (!ws || ws_bytes < plan.workspace_bytes || !aligned(ws, 16))
        return fail("dflash_verify_attention: workspace needs %zu bytes (16-byte aligned), got %zu",
                    plan.workspace_bytes, ws ? ws_bytes : (size_t)0);
    return hip_status(attn::launch_dflash_verify(p, &plan, scale, ring_k, ring_v, cur_q, cur_k, cur_v,
                                                 cache_lengths, write_positions, out, ws, (hipStream_t)stream),
                      "dflash_verify_attention");
}

int dflash_mask_rows(uint32_t lanes, uint32_t rows, uint32_t hidden, const uint16_t *mask_embedding,
                     float *draft_input, const uint64_t *bytes, void *stream) {
    if (lanes == 0 || lanes > 4 || rows < 2 || rows > 16 || hidden == 0)
        return fail("dflash_mask_rows: invalid DFlash2 mask-row geometry: DFlash2MaskRowsParams { lanes: %u, rows: "
                    "%u, hidden: %u }",
                    lanes, rows, hidden);
    const Need needs[] = {
        {"mask embedding", mask_embedding, hidden, 0, 0, 0, 2, 2},
        {"draft input", draft_input, (uint64_t)lanes * rows, hidden, 0, 0, 4, 4},
    };
    int st = check_buffers("dflash_mask_rows", needs, 2, bytes);
    if (st != ATTN_OK) return st;
    return hip_status(attn::launch_dflash_mask_rows(lanes, rows, hidden, mask_embedding, draft_input,
                                                    (hipStream_t)stream),
                      "dflash_mask_rows");
}

}  // extern "C"
