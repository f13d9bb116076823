// prepare.hip -- the step before paged attention on gfx950: per-head RMS norm
// of Q and K, rotary position embedding, and the K/V write into the pages.
//
// What is computed follows ferrum-kernels 0.8.3,
// src/backend/metal/vnext_ops/causal_attention.rs (the prepare dispatch: one
// threadgroup per (token, head slot) over query_heads + 2 * key_value_heads
// slots, reading the raw Q/K/V projections, the query and key norm weights,
// epsilon, rope_dim (even, at most head_dim), rope_theta, rope_interleaved
// and position_start, and writing the prepared query and the token's K/V
// into its page).  For token t of sequence b at position s = start_b + t:
//   x^ = x / sqrt(mean(x^2) + eps) * w           (Q and K heads; per head)
//   rotate pairs (x_a, x_b) of the first rope_dim features by s * theta^(-2i/rope_dim):
//     interleaved: pair i = (2i, 2i+1); otherwise pair i = (i, i + rope_dim/2)
//   Q -> q_out (f32), K -> k_pool, V (as is) -> v_pool at page
//   page_table[b][s / page_size], slot s % page_size.
//
// Design: one wave per (sequence, token, head slot), the head's features
// staged in LDS so any rotation pairing is one read; the work is a few KB per
// token, so the kernel is bound by launch and latency, not bandwidth.  The
// angle s * theta^(-2i/rope_dim) is formed and reduced modulo 2 pi in fp64:
// in f32 it would be off by about 1e-3 radians at positions of 16k.  The
// frequencies theta^(-2i/rope_dim) depend on i alone: the host computes them
// once, in fp64, and passes the table with the arguments.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kPrepareMaxPairs = 128;  // rope_dim <= head_dim <= 256

struct PrepareArgs {
    const float *q_raw, *k_raw, *v_raw, *q_norm, *k_norm;
    const int32_t *page_table, *query_lens, *position_starts;
    float *q_out;
    uint16_t *k_pool, *v_pool;
    int64_t qr_bs, qr_ts, qr_hs, kr_bs, kr_ts, kr_hs, vr_bs, vr_ts, vr_hs, qo_bs, qo_ts, qo_hs;
    int64_t qn_hs, kn_hs;  // norm weight head strides (0: one vector for every head)
    int64_t page_stride, token_stride, head_stride;
    int batch, n_heads, n_kv_heads, max_tokens, rope_dim, interleaved, use_norm;
    int page_size, max_pages, num_pages, ctx_cap;
    int bf16;
    float eps;
    double inv_freq[kPrepareMaxPairs];  // theta^(-2i/rope_dim), i < rope_dim / 2
};

constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr double kInvTwoPi = 0.15915494309189533576888376337251;

// Half a wave (32 lanes) per (sequence, token, head slot) item, two items per wave: lane
// l of a half holds features 4l + 128k .. 4l + 128k + 3 (k < D / 128), so the row is read
// and written with 16-byte accesses.  Every load that does not depend on another (the
// sequence's query length and start, the features, the norm weights) is issued before any
// is used; only the page entry waits for the start.
template <int D>
__global__ __launch_bounds__(256) void prepare_kernel(PrepareArgs a) {
    constexpr int NV = D / 128;  // float4 per lane
    __shared__ float s_x[8][D];  // one row per half wave
    const int lane = threadIdx.x & 63, l32 = lane & 31;
    const int half_id = threadIdx.x >> 5;  // 0..7 within the workgroup
    const int slots = a.n_heads + 2 * a.n_kv_heads;
    const int64_t items = (int64_t)a.batch * a.max_tokens * slots;
    const int64_t item = (int64_t)blockIdx.x * 8 + half_id;  // (b, t, slot)
    const bool live = item < items;
    const int64_t it = live ? item : items - 1;
    const int slot = (int)(it % slots);
    const int t = (int)((it / slots) % a.max_tokens);
    const int b = (int)(it / ((int64_t)slots * a.max_tokens));
    const bool is_q = slot < a.n_heads, is_k = !is_q && slot < a.n_heads + a.n_kv_heads;
    const int head = is_q ? slot : (is_k ? slot - a.n_heads : slot - a.n_heads - a.n_kv_heads);
    const int n_raw = a.query_lens[b];
    const int st_raw = a.position_starts[b];
    const float *src = is_q ? a.q_raw + b * a.qr_bs + (int64_t)t * a.qr_ts + (int64_t)head * a.qr_hs
                            : (is_k ? a.k_raw + b * a.kr_bs + (int64_t)t * a.kr_ts + (int64_t)head * a.kr_hs
                                    : a.v_raw + b * a.vr_bs + (int64_t)t * a.vr_ts + (int64_t)head * a.vr_hs);
    float4v x[NV], wn[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) x[k] = *reinterpret_cast<const float4v *>(src + 4 * l32 + 128 * k);
    const bool normed = (is_q || is_k) && a.use_norm;
    if (normed) {
        const float *w = is_q ? a.q_norm + (int64_t)head * a.qn_hs : a.k_norm + (int64_t)head * a.kn_hs;
#pragma unroll
        for (int k = 0; k < NV; ++k) wn[k] = *reinterpret_cast<const float4v *>(w + 4 * l32 + 128 * k);
    }
    const int n = n_raw < 0 ? 0 : (n_raw > a.max_tokens ? a.max_tokens : n_raw);
    const int st = st_raw < 0 ? 0 : st_raw;
    const int64_t pos64 = (int64_t)st + t;
    // this item is written: a live row of a new token, and for K/V within the pages the
    // sequence may use (every lane of a half wave agrees)
    const bool act = live && t < n && (is_q || pos64 < a.ctx_cap);

    if (is_q || is_k) {
        // the RMS sum runs over the 32 lanes of the half wave in every half, so that the
        // shuffles see their partners; inactive halves compute on their clamped item
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = fmaf(x[k][e], x[k][e], ss);
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        if (normed) {
            const float inv = 1.f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
            for (int k = 0; k < NV; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) x[k][e] = x[k][e] * inv * wn[k][e];
        }
        // rotary embedding; a split-halves partner comes from the half wave's LDS row
        if (!a.interleaved) {
#pragma unroll
            for (int k = 0; k < NV; ++k) *reinterpret_cast<float4v *>(&s_x[half_id][4 * l32 + 128 * k]) = x[k];
            __builtin_amdgcn_wave_barrier();  // LDS operations of one wave complete in order
        }
        const int half = a.rope_dim / 2;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            float4v y = x[k];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 4 * l32 + 128 * k + e;
                if (d < a.rope_dim) {
                    int i;
                    bool first;
                    float other;
                    if (a.interleaved) {
                        i = d >> 1;
                        first = (d & 1) == 0;
                        other = first ? x[k][e + 1 < 4 ? e + 1 : e] : x[k][e > 0 ? e - 1 : e];
                    } else {
                        first = d < half;
                        i = first ? d : d - half;
                        other = s_x[half_id][first ? d + half : d - half];
                    }
                    // angle = pos * theta^(-2i/rope_dim), reduced modulo 2 pi in fp64
                    const double ang = (double)pos64 * a.inv_freq[i];
                    const double red = ang - kTwoPi * floor(ang * kInvTwoPi);
                    float sn, cs;
                    sincosf((float)red, &sn, &cs);
                    y[e] = first ? x[k][e] * cs - other * sn : other * sn + x[k][e] * cs;
                }
            }
            x[k] = y;
        }
    }
    if (!act) return;

    if (is_q) {
        float *dst = a.q_out + b * a.qo_bs + (int64_t)t * a.qo_ts + (int64_t)head * a.qo_hs;
#pragma unroll
        for (int k = 0; k < NV; ++k) *reinterpret_cast<float4v *>(dst + 4 * l32 + 128 * k) = x[k];
        return;
    }
    const int pos = (int)pos64;  // below ctx_cap here
    const int pg = pos / a.page_size;
    int page = a.page_table[(int64_t)b * a.max_pages + pg];
    page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    uint16_t *pool = is_k ? a.k_pool : a.v_pool;
    uint16_t *dst = pool + (int64_t)page * a.page_stride + (int64_t)(pos - pg * a.page_size) * a.token_stride +
                    (int64_t)head * a.head_stride;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            h[e] = a.bf16 ? f32_to_bf16_rne(x[k][e]) : __builtin_bit_cast(uint16_t, (_Float16)x[k][e]);
        *reinterpret_cast<uint2 *>(dst + 4 * l32 + 128 * k) = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
    }
}

}  // namespace

hipError_t launch_paged_prepare(const attn_paged_prepare_params *p, const float *q_raw, const float *k_raw,
                                const float *v_raw, const float *q_norm, const float *k_norm,
                                const int32_t *page_table, const int32_t *query_lens,
                                const int32_t *position_starts, float *q_out, void *k_pool, void *v_pool,
                                hipStream_t stream) {
    PrepareArgs a;
    a.q_raw = q_raw;
    a.k_raw = k_raw;
    a.v_raw = v_raw;
    a.q_norm = q_norm;
    a.k_norm = k_norm;
    a.page_table = page_table;
    a.query_lens = query_lens;
    a.position_starts = position_starts;
    a.q_out = q_out;
    a.k_pool = (uint16_t *)k_pool;
    a.v_pool = (uint16_t *)v_pool;
    a.qr_bs = p->qr_bs;
    a.qr_ts = p->qr_ts;
    a.qr_hs = p->qr_hs;
    a.kr_bs = p->kr_bs;
    a.kr_ts = p->kr_ts;
    a.kr_hs = p->kr_hs;
    a.vr_bs = p->vr_bs;
    a.vr_ts = p->vr_ts;
    a.vr_hs = p->vr_hs;
    a.qo_bs = p->qo_bs;
    a.qo_ts = p->qo_ts;
    a.qo_hs = p->qo_hs;
    a.qn_hs = p->qn_hs;
    a.kn_hs = p->kn_hs;
    a.page_stride = p->kv_page_stride;
    a.token_stride = p->kv_token_stride;
    a.head_stride = p->kv_head_stride;
    a.batch = p->batch;
    a.n_heads = p->n_heads;
    a.n_kv_heads = p->n_kv_heads;
    a.max_tokens = p->max_tokens;
    a.rope_dim = p->rope_dim;
    a.interleaved = p->rope_interleaved != 0;
    a.use_norm = p->qk_norm != 0;
    a.page_size = p->page_size;
    a.max_pages = p->max_pages_per_seq;
    a.num_pages = p->num_pages;
    int cap = p->max_context;
    const int64_t table_cap = (int64_t)p->max_pages_per_seq * p->page_size;
    if (table_cap < cap) cap = (int)table_cap;
    a.ctx_cap = cap < 0 ? 0 : cap;
    a.bf16 = p->kv_dtype == ATTN_BF16;
    a.eps = p->epsilon;
    const double log2_theta = log2((double)p->rope_theta);
    for (int i = 0; i < kPrepareMaxPairs; ++i)
        a.inv_freq[i] = i < p->rope_dim / 2 ? exp2(-log2_theta * (2.0 * i) / (double)p->rope_dim) : 0.0;
    const int64_t items = (int64_t)p->batch * p->max_tokens * (p->n_heads + 2 * p->n_kv_heads);
    const dim3 grid((unsigned)((items + 7) / 8));  // eight half-wave items per workgroup
    switch (p->head_dim) {
    case 128: hipLaunchKernelGGL((prepare_kernel<128>), grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL((prepare_kernel<256>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace attn
