// decode.hip -- single-query attention over a paged KV cache on gfx950.
//
// What is computed follows ferrum-kernels 0.8.3,
// src/backend/metal/vnext_ops/causal_attention.rs (the attention dispatch
// over fixed-size KV pages read through a per-sequence page table; query head
// h reads KV head h / (query_heads / key_value_heads); the context includes
// the token the step wrote).
//
// Design: decode is bound by HBM reads of K and V, so the kernel maximises
// bytes in flight rather than arithmetic rate.
//  * Split-KV: workgroup (split, KV head, sequence) walks `chunk` tokens of
//    one sequence for all query heads of one KV head (the K/V rows are read
//    once for the whole group), then a second kernel merges the splits with a
//    log-sum-exp reduction.
//  * Inside a workgroup, 16 groups of 16 lanes each walk their own tokens;
//    one token row (head_dim f16) is spread over the 16 lanes of a group as
//    128-bit loads, so a row of 256 bytes is one coalesced access.  Each
//    group keeps its own online-softmax state; scores are reduced across the
//    16 lanes with DPP row operations.  The 16 group states are merged in LDS
//    at the end of the chunk.
//  * Every lane has 2*TB row loads in flight per step (TB tokens, K and V).
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;
constexpr int kGroups = kThreads / 16;

struct DecodeArgs {
    const float *q;
    const uint16_t *k_pool, *v_pool;
    const int32_t *page_table, *context_lens;
    float *o;
    float *part;
    float2 *ml;
    int64_t q_bs, q_hs, o_bs, o_hs, page_stride, token_stride, head_stride;
    int batch, n_heads, group, heads_per_wg, page_size, max_pages, num_pages, ctx_cap;
    int chunk, max_splits;
    float score_scale;
};

template <bool BF16>
__device__ __forceinline__ float kv_to_f32(uint32_t word, int hi) {
    const uint16_t x = hi ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xffffu);
    if constexpr (BF16) {
        return bf16_bits_to_f32(x);
    } else {
        return f16_bits_to_f32(x);
    }
}

__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

template <int D, int GW, bool BF16>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecodeArgs a) {
    constexpr int VPL = D / 16;            // elements of a row per lane
    constexpr int TB = D <= 128 ? 8 : 4;   // tokens per group per step
    constexpr int W4 = VPL / 8;            // 128-bit words per lane per row

    const int split = blockIdx.x;
    const int hsplit = a.group / GW;
    const int kvh = blockIdx.y / hsplit;
    const int head0 = kvh * a.group + (blockIdx.y % hsplit) * GW;
    const int b = blockIdx.z;
    const int ctx = clamp_ctx(a.context_lens[b], a.ctx_cap);
    const int t0 = split * a.chunk;
    const int64_t unit0 = (int64_t)b * a.n_heads + head0;
    if (t0 >= ctx) {
        if (threadIdx.x < GW) a.ml[(unit0 + threadIdx.x) * a.max_splits + split] = make_float2(-INFINITY, 0.f);
        return;
    }
    const int t1 = t0 + a.chunk < ctx ? t0 + a.chunk : ctx;

    const int grp = threadIdx.x >> 4;
    const int sub = threadIdx.x & 15;

    float q[GW][VPL];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
        const float *qp = a.q + b * a.q_bs + (int64_t)(head0 + hh) * a.q_hs + sub * VPL;
#pragma unroll
        for (int i = 0; i < VPL; i += 4) {
            const float4v x = *reinterpret_cast<const float4v *>(qp + i);
#pragma unroll
            for (int e = 0; e < 4; ++e) q[hh][i + e] = x[e] * a.score_scale;
        }
    }
    float m[GW], l[GW], o[GW][VPL];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
        m[hh] = -INFINITY;
        l[hh] = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) o[hh][i] = 0.f;
    }

    const int32_t *pt = a.page_table + (int64_t)b * a.max_pages;
    const int64_t head_off = (int64_t)kvh * a.head_stride + sub * VPL;

    for (int base = t0 + grp * TB; base < t1; base += kGroups * TB) {
        uint4v kw[TB][W4], vw[TB][W4];
#pragma unroll
        for (int k = 0; k < TB; ++k) {
            const int t = base + k;
            if (t < t1) {
                int page = pt[t / a.page_size];
                page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
                const int64_t off = (int64_t)page * a.page_stride + (int64_t)(t % a.page_size) * a.token_stride + head_off;
#pragma unroll
                for (int w = 0; w < W4; ++w) {
                    kw[k][w] = *reinterpret_cast<const uint4v *>(a.k_pool + off + 8 * w);
                    vw[k][w] = *reinterpret_cast<const uint4v *>(a.v_pool + off + 8 * w);
                }
            } else {
#pragma unroll
                for (int w = 0; w < W4; ++w) {
                    kw[k][w] = uint4v{0u, 0u, 0u, 0u};
                    vw[k][w] = kw[k][w];
                }
            }
        }
        float sc[GW][TB];
#pragma unroll
        for (int k = 0; k < TB; ++k) {
            float kf[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) kf[i] = kv_to_f32<BF16>(kw[k][i / 8][(i % 8) / 2], i & 1);
#pragma unroll
            for (int hh = 0; hh < GW; ++hh) {
                float s = 0.f;
#pragma unroll
                for (int i = 0; i < VPL; ++i) s = fmaf(q[hh][i], kf[i], s);
                s = row16_sum(s);
                sc[hh][k] = base + k < t1 ? s : -INFINITY;
            }
        }
#pragma unroll
        for (int hh = 0; hh < GW; ++hh) {
            float mx = m[hh];
#pragma unroll
            for (int k = 0; k < TB; ++k) mx = fmaxf(mx, sc[hh][k]);
            const float alpha = exp2f(m[hh] - mx);  // mx is finite: the first token of this step is real
            m[hh] = mx;
            float p[TB];
            float ps = 0.f;
#pragma unroll
            for (int k = 0; k < TB; ++k) {
                p[k] = exp2f(sc[hh][k] - mx);
                ps += p[k];
            }
            l[hh] = l[hh] * alpha + ps;
#pragma unroll
            for (int i = 0; i < VPL; ++i) o[hh][i] *= alpha;
#pragma unroll
            for (int k = 0; k < TB; ++k)
#pragma unroll
                for (int i = 0; i < VPL; ++i) o[hh][i] = fmaf(p[k], kv_to_f32<BF16>(vw[k][i / 8][(i % 8) / 2], i & 1), o[hh][i]);
        }
    }

    // ---- merge the 16 group states of this workgroup through LDS
    __shared__ float s_o[kGroups][GW][D];
    __shared__ float s_ml[kGroups][GW][2];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) s_o[grp][hh][sub * VPL + i] = o[hh][i];
        if (sub == 0) {
            s_ml[grp][hh][0] = m[hh];
            s_ml[grp][hh][1] = l[hh];
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < GW * D; e += kThreads) {
        const int hh = e / D, d = e % D;
        float mmax = -INFINITY;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) mmax = fmaxf(mmax, s_ml[g][hh][0]);
        float acc = 0.f, lsum = 0.f;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            const float mg = s_ml[g][hh][0];
            if (mg == -INFINITY) continue;  // group walked no token
            const float w = exp2f(mg - mmax);
            acc = fmaf(w, s_o[g][hh][d], acc);
            lsum = fmaf(w, s_ml[g][hh][1], lsum);
        }
        const int64_t u = (unit0 + hh) * a.max_splits + split;
        a.part[u * D + d] = acc;
        if (d == 0) a.ml[u] = make_float2(mmax, lsum);
    }
}

// One thread per 4 output elements: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
    constexpr int PER_UNIT = D / 4;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t unit = t / PER_UNIT;
    const int d4 = t % PER_UNIT;
    if (unit >= (int64_t)a.batch * a.n_heads) return;
    const int b = unit / a.n_heads, head = unit % a.n_heads;
    const int ctx = clamp_ctx(a.context_lens[b], a.ctx_cap);
    int nsplit = (ctx + a.chunk - 1) / a.chunk;
    if (nsplit > a.max_splits) nsplit = a.max_splits;
    const float2 *ml = a.ml + unit * a.max_splits;
    float mmax = -INFINITY;
    for (int s = 0; s < nsplit; ++s) mmax = fmaxf(mmax, ml[s].x);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    if (mmax != -INFINITY) {
        for (int s = 0; s < nsplit; ++s) {
            if (ml[s].x == -INFINITY) continue;
            const float w = exp2f(ml[s].x - mmax);
            lsum += w * ml[s].y;
            acc += w * *reinterpret_cast<const float4v *>(a.part + (unit * a.max_splits + s) * D + 4 * d4);
        }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    *reinterpret_cast<float4v *>(a.o + b * a.o_bs + (int64_t)head * a.o_hs + 4 * d4) = acc * inv;
}

template <int D, int GW, bool BF16>
hipError_t launch_typed(const DecodeArgs &a, hipStream_t stream) {
    dim3 grid(a.max_splits, (a.n_heads / a.group) * (a.group / GW), a.batch);
    hipLaunchKernelGGL((decode_partial_kernel<D, GW, BF16>), grid, dim3(kThreads), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t threads = (int64_t)a.batch * a.n_heads * (D / 4);
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_gw(const DecodeArgs &a, hipStream_t stream) {
    switch (a.heads_per_wg) {
    case 1: return launch_typed<D, 1, BF16>(a, stream);
    case 2: return launch_typed<D, 2, BF16>(a, stream);
    case 4: return launch_typed<D, 4, BF16>(a, stream);
    case 8:
        if constexpr (D <= 128) return launch_typed<D, 8, BF16>(a, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int plan_decode(const attn_decode_params *p, DecodePlan *plan) {
    plan->head_dim = p->head_dim;
    plan->group = p->n_heads / p->n_kv_heads;
    const int max_gw = p->head_dim <= 128 ? 8 : 4;
    int gw = 1;
    for (int c = 1; c <= max_gw; c *= 2)
        if (plan->group % c == 0) gw = c;
    plan->heads_per_wg = gw;
    int cap = p->max_context;
    const int64_t table_cap = (int64_t)p->max_pages_per_seq * p->page_size;
    if (table_cap < cap) cap = (int)table_cap;
    plan->chunk = cap <= 2048 ? 128 : (cap <= 8192 ? 256 : 512);
    plan->max_splits = cap > 0 ? (cap + plan->chunk - 1) / plan->chunk : 1;
    const size_t units = (size_t)p->batch * p->n_heads;
    plan->ml_offset = 0;
    plan->ml_bytes = units * plan->max_splits * sizeof(float2);
    plan->part_offset = (plan->ml_bytes + 255) & ~(size_t)255;
    plan->part_bytes = units * plan->max_splits * p->head_dim * sizeof(float);
    plan->workspace_bytes = plan->part_offset + plan->part_bytes;
    return ATTN_OK;
}

hipError_t launch_paged_decode(const attn_decode_params *p, const DecodePlan *plan, const float *q,
                               const void *k_pool, const void *v_pool, const int32_t *page_table,
                               const int32_t *context_lens, float *o, void *ws, hipStream_t stream) {
    DecodeArgs a;
    a.q = q;
    a.k_pool = (const uint16_t *)k_pool;
    a.v_pool = (const uint16_t *)v_pool;
    a.page_table = page_table;
    a.context_lens = context_lens;
    a.o = o;
    a.ml = (float2 *)((uint8_t *)ws + plan->ml_offset);
    a.part = (float *)((uint8_t *)ws + plan->part_offset);
    a.q_bs = p->q_bs;
    a.q_hs = p->q_hs;
    a.o_bs = p->o_bs;
    a.o_hs = p->o_hs;
    a.page_stride = p->kv_page_stride;
    a.token_stride = p->kv_token_stride;
    a.head_stride = p->kv_head_stride;
    a.batch = p->batch;
    a.n_heads = p->n_heads;
    a.group = plan->group;
    a.heads_per_wg = plan->heads_per_wg;
    a.page_size = p->page_size;
    a.max_pages = p->max_pages_per_seq;
    a.num_pages = p->num_pages;
    int cap = p->max_context;
    const int64_t table_cap = (int64_t)p->max_pages_per_seq * p->page_size;
    if (table_cap < cap) cap = (int)table_cap;
    a.ctx_cap = cap;
    a.chunk = plan->chunk;
    a.max_splits = plan->max_splits;
    a.score_scale = p->scale * kLog2e;
    const bool bf16 = p->kv_dtype == ATTN_BF16;
    switch (p->head_dim) {
    case 128: return bf16 ? launch_gw<128, true>(a, stream) : launch_gw<128, false>(a, stream);
    case 256: return bf16 ? launch_gw<256, true>(a, stream) : launch_gw<256, false>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
