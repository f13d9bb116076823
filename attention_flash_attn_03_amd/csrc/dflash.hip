// dflash.hip -- DFlash2 block-verify ring steps for gfx950: pack, mask,
// commit and mask-rows.  All four are bandwidth-bound gather/scatter work:
// one thread moves one 16-byte chunk (8 bf16 elements) so every global
// access is a 128-bit load or store on a contiguous row.
//
// Semantics follow mlx-native 0.21.1, src/ops/dflash2_attention_pack.rs
// (the kernel table, the dispatch functions' buffer shapes and the test
// gpu_pack_mask_and_commit_match_ring_semantics).
#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint4v load_f32x8_as_bf16(const float *src) {
    const float4v a = *reinterpret_cast<const float4v *>(src);
    const float4v b = *reinterpret_cast<const float4v *>(src + 4);
    uint4v out;
    out[0] = pack2(f32_to_bf16_rne(a[0]), f32_to_bf16_rne(a[1]));
    out[1] = pack2(f32_to_bf16_rne(a[2]), f32_to_bf16_rne(a[3]));
    out[2] = pack2(f32_to_bf16_rne(b[0]), f32_to_bf16_rne(b[1]));
    out[3] = pack2(f32_to_bf16_rne(b[2]), f32_to_bf16_rne(b[3]));
    return out;
}

// Threads [0, nq) pack Q chunks; threads [nq, nq + nkv) pack K and V chunks.
__global__ __launch_bounds__(kThreads) void pack_kernel(
    dflash_params p, const uint16_t *__restrict__ ring_k, const uint16_t *__restrict__ ring_v,
    const float *__restrict__ cur_q, const float *__restrict__ cur_k, const float *__restrict__ cur_v,
    const uint32_t *__restrict__ cache_lengths, const uint32_t *__restrict__ write_positions,
    uint16_t *__restrict__ packed_q, uint16_t *__restrict__ packed_k, uint16_t *__restrict__ packed_v,
    uint64_t nq, uint64_t nkv) {
    const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    const uint32_t chunks = p.head_dim / 8;
    if (t < nq) {
        const uint32_t dc = t % chunks;
        uint64_t rest = t / chunks;
        const uint32_t i = rest % p.rows;
        rest /= p.rows;
        const uint32_t h = rest % p.q_heads;
        const uint64_t b = rest / p.q_heads;
        const float *src = cur_q + ((b * p.rows + i) * p.q_heads + h) * p.head_dim + dc * 8;
        uint16_t *dst = packed_q + ((b * p.q_heads + h) * p.rows + i) * p.head_dim + dc * 8;
        *reinterpret_cast<uint4v *>(dst) = load_f32x8_as_bf16(src);
        return;
    }
    if (t >= nq + nkv) return;
    const uint64_t u = t - nq;
    const uint32_t dc = u % chunks;
    uint64_t rest = u / chunks;
    const uint32_t pos = rest % p.packed_len;
    rest /= p.packed_len;
    const uint32_t kh = rest % p.kv_heads;
    const uint64_t b = rest / p.kv_heads;
    const uint64_t dst_off = ((b * p.kv_heads + kh) * p.packed_len + pos) * p.head_dim + dc * 8;
    uint4v kval, vval;
    if (pos < p.rows) {
        // drafted rows first, in order
        const uint64_t src = ((b * p.rows + pos) * p.kv_heads + kh) * p.head_dim + dc * 8;
        kval = load_f32x8_as_bf16(cur_k + src);
        vval = load_f32x8_as_bf16(cur_v + src);
    } else {
        // then the cache, newest first: j-th newest row is ring slot (wp - 1 - j) mod w;
        // the lane's length and write position are requested together
        const uint32_t j = pos - p.rows;
        const uint32_t length = cache_lengths[b];
        const uint32_t wp = write_positions[b] % p.window;
        if (j < length) {
            const uint32_t slot = (wp + p.window - 1 - j) % p.window;
            const uint64_t src = ((b * p.kv_heads + kh) * p.window + slot) * p.head_dim + dc * 8;
            kval = *reinterpret_cast<const uint4v *>(ring_k + src);
            vval = *reinterpret_cast<const uint4v *>(ring_v + src);
        } else {
            kval = uint4v{0u, 0u, 0u, 0u};
            vval = kval;
        }
    }
    *reinterpret_cast<uint4v *>(packed_k + dst_off) = kval;
    *reinterpret_cast<uint4v *>(packed_v + dst_off) = vval;
}

// One thread writes 8 consecutive mask elements of the flat [b, h, r, k] array.  The
// first element's (lane, head, row, position) is found once, with 32-bit index
// arithmetic whenever the array has fewer than 2^32 elements (integer division is a
// long instruction sequence on the GPU, and 64-bit division far longer); the other
// seven follow by stepping the position and carrying into row, head and lane.
template <typename IDX>
__global__ __launch_bounds__(kThreads) void mask_kernel(dflash_params p,
                                                        const uint32_t *__restrict__ cache_lengths,
                                                        uint16_t *__restrict__ mask, uint64_t total) {
    const uint64_t first = ((uint64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
    if (first >= total) return;
    const IDX f = (IDX)first;
    const IDX row = f / (IDX)p.packed_len;               // flat (lane, head, row) index
    uint32_t pos = (uint32_t)(f - row * (IDX)p.packed_len);
    const IDX bh = row / (IDX)p.rows;
    uint32_t i = (uint32_t)(row - bh * (IDX)p.rows);
    uint32_t h = (uint32_t)(bh % (IDX)p.q_heads);
    uint32_t b = (uint32_t)(bh / (IDX)p.q_heads);
    auto reach_of = [&](uint32_t bb, uint32_t ii) {
        const uint32_t length = bb < p.lanes ? cache_lengths[bb] : 0u;
        const uint32_t window_reach = p.window - 1 - ii;
        return length < window_reach ? length : window_reach;
    };
    uint32_t reach = reach_of(b, i);
    uint16_t vals[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool visible = pos < p.rows || (pos - p.rows) < reach;
        vals[e] = visible ? (uint16_t)0x0000 : (uint16_t)0xFF80;
        if (++pos == p.packed_len) {
            pos = 0;
            if (++i == p.rows) {
                i = 0;
                if (++h == p.q_heads) {
                    h = 0;
                    ++b;
                }
            }
            reach = reach_of(b, i);
        }
    }
    if (first + 8 <= total) {
        uint4v out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = pack2(vals[2 * e], vals[2 * e + 1]);
        *reinterpret_cast<uint4v *>(mask + first) = out;
    } else {
        for (uint64_t e = 0; first + e < total; ++e) mask[first + e] = vals[e];
    }
}

// One thread per committed 8-element chunk.  Its indices come from 32-bit arithmetic when
// the chunks number fewer than 2^32 (IDX = uint32_t); the commit count, the write position
// and the new row are requested together (the row exists for every c < max_commit), so the
// call is one memory round trip before the stores.
template <typename IDX>
__global__ __launch_bounds__(kThreads) void commit_kernel(
    dflash_params p, const float *__restrict__ new_k, const float *__restrict__ new_v,
    const uint32_t *__restrict__ commit_counts, const uint32_t *__restrict__ write_positions,
    uint16_t *__restrict__ ring_k, uint16_t *__restrict__ ring_v, uint64_t total) {
    const uint64_t t64 = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t64 >= total) return;
    const IDX t = (IDX)t64;
    const uint32_t chunks = p.head_dim / 8;
    const uint32_t dc = (uint32_t)(t % chunks);
    IDX rest = t / chunks;
    const uint32_t kh = (uint32_t)(rest % p.kv_heads);
    rest /= p.kv_heads;
    const uint32_t c = (uint32_t)(rest % p.max_commit);
    const uint64_t b = (uint64_t)(rest / p.max_commit);
    const uint32_t n_raw = commit_counts[b];
    const uint32_t wp = write_positions[b];
    const uint64_t src = ((b * p.max_commit + c) * p.kv_heads + kh) * p.head_dim + dc * 8;
    const uint4v kval = load_f32x8_as_bf16(new_k + src);
    const uint4v vval = load_f32x8_as_bf16(new_v + src);
    const uint32_t n = n_raw > p.max_commit ? p.max_commit : n_raw;
    if (c >= n) return;
    const uint32_t slot = (uint32_t)(((uint64_t)(wp % p.window) + c) % p.window);
    const uint64_t dst = ((b * p.kv_heads + kh) * p.window + slot) * p.head_dim + dc * 8;
    *reinterpret_cast<uint4v *>(ring_k + dst) = kval;
    *reinterpret_cast<uint4v *>(ring_v + dst) = vval;
}

__global__ __launch_bounds__(kThreads) void mask_rows_kernel(uint32_t rows, uint32_t hidden,
                                                             const uint16_t *__restrict__ embedding,
                                                             float *__restrict__ draft, uint64_t total) {
    const uint64_t t = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= total) return;
    const uint32_t x = t % hidden;
    const uint64_t rest = t / hidden;
    const uint32_t i = 1 + rest % (rows - 1);  // row 0 of each lane is the anchor
    const uint64_t b = rest / (rows - 1);
    draft[(b * rows + i) * hidden + x] = bf16_bits_to_f32(embedding[x]);
}

inline unsigned blocks_for(uint64_t threads) { return (unsigned)((threads + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_dflash_pack(const dflash_params *p, const uint16_t *ring_k, const uint16_t *ring_v,
                              const float *cur_q, const float *cur_k, const float *cur_v,
                              const uint32_t *cache_lengths, const uint32_t *write_positions,
                              uint16_t *packed_q, uint16_t *packed_k, uint16_t *packed_v,
                              hipStream_t stream) {
    const uint64_t chunks = p->head_dim / 8;
    const uint64_t nq = (uint64_t)p->lanes * p->q_heads * p->rows * chunks;
    const uint64_t nkv = (uint64_t)p->lanes * p->kv_heads * p->packed_len * chunks;
    hipLaunchKernelGGL(pack_kernel, dim3(blocks_for(nq + nkv)), dim3(kThreads), 0, stream, *p, ring_k,
                       ring_v, cur_q, cur_k, cur_v, cache_lengths, write_positions, packed_q, packed_k,
                       packed_v, nq, nkv);
    return hipGetLastError();
}

hipError_t launch_dflash_mask(const dflash_params *p, const uint32_t *cache_lengths, uint16_t *mask,
                              hipStream_t stream) {
    const uint64_t total = (uint64_t)p->lanes * p->q_heads * p->rows * p->packed_len;
    if (total < ((uint64_t)1 << 32)) {
        hipLaunchKernelGGL(mask_kernel<uint32_t>, dim3(blocks_for((total + 7) / 8)), dim3(kThreads), 0, stream, *p,
                           cache_lengths, mask, total);
    } else {
        hipLaunchKernelGGL(mask_kernel<uint64_t>, dim3(blocks_for((total + 7) / 8)), dim3(kThreads), 0, stream, *p,
                           cache_lengths, mask, total);
    }
    return hipGetLastError();
}

hipError_t launch_dflash_commit(const dflash_params *p, const float *new_k, const float *new_v,
                                const uint32_t *commit_counts, const uint32_t *write_positions,
                                uint16_t *ring_k, uint16_t *ring_v, hipStream_t stream) {
    const uint64_t total = (uint64_t)p->lanes * p->max_commit * p->kv_heads * (p->head_dim / 8);
    if (total < ((uint64_t)1 << 32)) {
        hipLaunchKernelGGL(commit_kernel<uint32_t>, dim3(blocks_for(total)), dim3(kThreads), 0, stream, *p, new_k,
                           new_v, commit_counts, write_positions, ring_k, ring_v, total);
    } else {
        hipLaunchKernelGGL(commit_kernel<uint64_t>, dim3(blocks_for(total)), dim3(kThreads), 0, stream, *p, new_k,
                           new_v, commit_counts, write_positions, ring_k, ring_v, total);
    }
    return hipGetLastError();
}

hipError_t launch_dflash_mask_rows(uint32_t lanes, uint32_t rows, uint32_t hidden,
                                   const uint16_t *mask_embedding, float *draft_input,
                                   hipStream_t stream) {
    const uint64_t total = (uint64_t)lanes * (rows - 1) * hidden;
    hipLaunchKernelGGL(mask_rows_kernel, dim3(blocks_for(total)), dim3(kThreads), 0, stream, rows, hidden,
                       mask_embedding, draft_input, total);
    return hipGetLastError();
}

}  // namespace attn
