// prefill.hip -- masked grouped-query attention forward on gfx950 MFMA.
//
// What is computed follows mlx-native 0.18.0, src/ops/flash_attn_prefill_tensor.rs
// (module header, FlashAttnPrefillTensorParams): O = softmax(scale Q K^T + mask) V
// with an online softmax over 64-row KV tiles, one KV head per
// n_heads/n_kv_heads query heads, an additive mask whose (query block, KV
// tile) blocks are classified beforehand so empty tiles are skipped.
//
// CDNA4 design (not the page's Metal design):
//  * A wave owns 32 query slots (query row, head pairs of one KV head) and the
//    whole head dimension.  It computes S^T = K Q^T with
//    v_mfma_f32_32x32x16_{f16,bf16}: the accumulator layout puts one query
//    column in each lane (lane l holds query l%32 and 16 keys of a 32-key
//    block), so row max / row sum are in-lane plus one permlane32 swap, and
//    the rescale of the output is a per-lane scalar.  O^T for head_dim 512
//    lives in the 256 accumulation registers (one wave per SIMD).
//  * O^T = V^T P^T reuses P^T straight from the S^T accumulator registers as
//    the B operand; V stays row-major in LDS and its transposed A fragments
//    come from ds_read_b64_tr_b16 (4 keys x 1 column per lane per read).
//  * K and V tiles (64 rows) stream into LDS with global_load_lds_dwordx4
//    (no staging registers), XOR-swizzled so both LDS read patterns are free
//    of bank conflicts.  The loads are offset by half a tile: K(j+1) lands
//    while softmax and P V of tile j run, V(j+1) while S of tile j+1 runs.
//  * exp2 with log2(e) folded into the score scale; P is rounded to the K/V
//    type before P V and the running sum l is taken from the rounded P, so
//    the rounding cancels in O / l.  O is rescaled only when some lane's
//    running max moved (lazy rescale).
//  * Row blocks are dispatched longest first (causal frontiers make the last
//    blocks the heaviest).  Optional KV split across workgroups with a
//    log-sum-exp combine pass for calls with few query blocks (block verify).
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr int kTile = 64;               // KV rows per step
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Geo {
    static constexpr int CH = D / 8;         // 16-byte chunks per K/V row
    static constexpr int KSTEPS = D / 16;    // MFMA k-steps for S
    static constexpr int DBLK = D / 32;      // 32-column O blocks per wave
    static constexpr int TILE_ELEMS = kTile * D;
};

struct PrefillArgs {
    const void *q, *k, *v, *mask;
    float *o;
    const uint8_t *blk;
    float *part;       // split partials (unnormalised O)
    float2 *ml;        // split partials (running max in log2 units, running sum)
    int64_t q_bs, q_rs, q_hs, k_bs, k_rs, k_hs, v_bs, v_rs, v_hs, m_bs, m_hs, m_rs, o_bs, o_rs, o_hs;
    int batch, rows, kv_len, n_heads, group;
    int rows_per_wg, heads_per_wg, row_blocks, head_groups, blk_heads;
    int kv_tiles, blk_stride, splits, tiles_per_split;
    int q_bf16, mask_bf16, mask_vec;
    float score_scale;  // scale * log2(e)
};

template <bool BF16>
__device__ __forceinline__ float16v mfma32(uint4v a, uint4v b, float16v c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bhalf8, a), __builtin_bit_cast(bhalf8, b),
                                                       c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c,
                                                      0, 0, 0);
    }
}

template <bool BF16>
__device__ __forceinline__ uint16_t to_kv16(float x) {
    if constexpr (BF16) {
        return f32_to_bf16_rne(x);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
}

template <bool BF16>
__device__ __forceinline__ float from_kv16(uint16_t x) {
    if constexpr (BF16) {
        return bf16_bits_to_f32(x);
    } else {
        return f16_bits_to_f32(x);
    }
}

typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

__device__ __forceinline__ short4v read_tr16(const uint16_t *lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(lds_ptr));
}

// LDS tile layouts (64 rows x D, no padding).  Chunk = 16 bytes = 8 elements.
//  K: logical chunk c of row r sits at physical chunk c ^ (r % 16); the S^T
//     A-operand read (16 consecutive rows, one chunk) hits 16 distinct banks.
//  V: logical chunk c of row r sits at physical chunk c ^ 4*(r % 4); the
//     transposing read (4 consecutive rows x 4 chunks per 32 lanes) hits 16
//     distinct bank groups.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 2; }

// Stream one 64-row tile of K or V into LDS with global_load_lds_dwordx4: a
// wave-instruction fills 64 consecutive 16-byte LDS slots starting at M0, so
// each lane fetches the global chunk that belongs in its slot.  Rows past
// kv_len fetch row kv_len-1 (finite data; those keys are masked to -inf).
// Every wave issues exactly NLD instructions; the explicit vmcnt waits below
// count them.  The instruction is issued from inline asm so the compiler does
// not treat every later LDS read as dependent on it (its conservative
// vmcnt(0) would drain the prefetch of the other tile); its own waits for
// other loads only get stricter, never weaker, from loads it cannot see.
template <int D, int NW, bool IS_V>
__device__ __forceinline__ void issue_tile(uint16_t *lds, const uint16_t *base, int64_t row_stride, int key0,
                                           int kv_len, int wave, int lane) {
    constexpr int CH = D / 8;
    constexpr int NLD = kTile * CH / (64 * NW);
    // recompute the per-lane addresses here instead of keeping 2*NLD of them live across the loop
    asm volatile("" : "+v"(lane));
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void *)lds;
#pragma unroll
    for (int it = 0; it < NLD; ++it) {
        const int slot0 = (it * NW + wave) * 64;
        const int slot = slot0 + lane;
        const int row = slot / CH;
        const int pch = slot % CH;
        const int ch = pch ^ (IS_V ? v_swz(row) : k_swz(row));
        int grow = key0 + row;
        grow = grow < kv_len ? grow : kv_len - 1;
        const uint16_t *src = base + (int64_t)grow * row_stride + ch * 8;
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base + slot0 * 16);
        // M0 is a reserved register the compiler does not let inline asm clobber; nothing
        // else in this kernel reads it (no movrel, sendmsg or LDS-DMA intrinsic), so writing
        // it here is safe.
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory");
    }
}

// Wait until at most N of this wave's vector-memory operations are in flight,
// then meet the other waves.  Loads retire in order, so N = the count issued
// after the ones we need.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_done_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef const __attribute__((address_space(4))) uint32_t const_u32;

// QSPLIT: f32 Q against bf16 K/V.  bf16 keeps 8 significant bits, which
// perturbs every score by about 2^-9 relative; Q is carried as hi + lo bf16
// parts (about 16 significant bits) and both products go into S.
//
// NW waves per workgroup; with head_dim 512 the waves pair up as two slices
// of 256 head-dim columns over the same 32 query slots (NS = 2) and add their
// partial scores through LDS; otherwise every wave has its own query slots.
template <int D, int NW, bool BF16, bool HAS_MASK, bool QSPLIT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_kernel(PrefillArgs a) {
    using G = Geo<D>;
    constexpr int NS = D > 256 ? 2 : 1;       // head-dim slices
    constexpr int DS = D / NS;                 // columns per wave
    constexpr int KSTEPS = DS / 16;            // MFMA k-steps of S over a slice
    constexpr int DBLK = DS / 32;              // 32-column O blocks per wave
    constexpr int NLD = kTile * G::CH / (64 * NW);
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds[G::TILE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds[G::TILE_ELEMS];
    __shared__ __attribute__((aligned(16))) float x_lds[NS > 1 ? NW * 2 * 16 * 64 : 1];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int slice = wave % NS;
    const int qwave = wave / NS;
    const int half = lane >> 5;    // which 8-element k half of an MFMA operand this lane feeds
    const int col = lane & 31;     // query slot column inside the wave

    // longest-first: with a causal frontier the last row blocks carry the most tiles
    const int rb = a.row_blocks - 1 - (int)blockIdx.x;
    const int hg = blockIdx.y;
    const int b = blockIdx.z / a.splits;
    const int split = blockIdx.z % a.splits;
    const int h0 = hg * a.heads_per_wg;
    const int kvh = h0 / a.group;

    // this lane's query slot
    const int slot = qwave * 32 + col;
    const int head = h0 + slot / a.rows_per_wg;
    const int row = rb * a.rows_per_wg + slot % a.rows_per_wg;
    const bool row_ok = row < a.rows;
    const int row_c = row_ok ? row : a.rows - 1;

    // ---- Q fragment: B operand of S^T = K Q^T, k = slice*DS + 16*ks + 8*half + i
    uint4v qf[KSTEPS];
    uint4v qlo[QSPLIT ? KSTEPS : 1];
    {
        const int dbase = slice * DS + 8 * half;
        if (a.q_bf16) {
            const uint16_t *qp = (const uint16_t *)a.q + b * a.q_bs + (int64_t)row_c * a.q_rs + head * a.q_hs + dbase;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                uint4v raw = *reinterpret_cast<const uint4v *>(qp + 16 * ks);
                if constexpr (BF16) {
                    qf[ks] = raw;
                } else {
                    uint4v cv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float lo = bf16_bits_to_f32((uint16_t)(raw[e] & 0xffffu));
                        const float hi = bf16_bits_to_f32((uint16_t)(raw[e] >> 16));
                        cv[e] = pack2(to_kv16<false>(lo), to_kv16<false>(hi));
                    }
                    qf[ks] = cv;
                }
            }
        } else {
            const float *qp = (const float *)a.q + b * a.q_bs + (int64_t)row_c * a.q_rs + head * a.q_hs + dbase;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const float4v x0 = *reinterpret_cast<const float4v *>(qp + 16 * ks);
                const float4v x1 = *reinterpret_cast<const float4v *>(qp + 16 * ks + 4);
                uint4v cv;
                cv[0] = pack2(to_kv16<BF16>(x0[0]), to_kv16<BF16>(x0[1]));
                cv[1] = pack2(to_kv16<BF16>(x0[2]), to_kv16<BF16>(x0[3]));
                cv[2] = pack2(to_kv16<BF16>(x1[0]), to_kv16<BF16>(x1[1]));
                cv[3] = pack2(to_kv16<BF16>(x1[2]), to_kv16<BF16>(x1[3]));
                qf[ks] = cv;
                if constexpr (QSPLIT) {
                    float rest[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        rest[e] = x0[e] - bf16_bits_to_f32((uint16_t)(cv[e / 2] >> (16 * (e & 1))));
                        rest[4 + e] = x1[e] - bf16_bits_to_f32((uint16_t)(cv[2 + e / 2] >> (16 * (e & 1))));
                    }
                    qlo[ks] = uint4v{pack2(f32_to_bf16_rne(rest[0]), f32_to_bf16_rne(rest[1])),
                                     pack2(f32_to_bf16_rne(rest[2]), f32_to_bf16_rne(rest[3])),
                                     pack2(f32_to_bf16_rne(rest[4]), f32_to_bf16_rne(rest[5])),
                                     pack2(f32_to_bf16_rne(rest[6]), f32_to_bf16_rne(rest[7]))};
                }
            }
        }
        if (!row_ok) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                qf[ks] = uint4v{0u, 0u, 0u, 0u};
                if constexpr (QSPLIT) qlo[ks] = qf[ks];
            }
        }
    }

    const uint16_t *mrow = nullptr;
    if constexpr (HAS_MASK) {
        mrow = (const uint16_t *)a.mask + b * a.m_bs + head * a.m_hs + (int64_t)row_c * a.m_rs;
    }

    float16v acc_o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_run = -INFINITY;  // running max of the log2-scaled scores
    float l_run = 0.f;        // running sum of the rounded probabilities

    const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_bs + kvh * a.k_hs;
    const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_bs + kvh * a.v_hs;
    // tile codes are read as dwords through the scalar cache (constant address space)
    const_u32 *blk_row = nullptr;
    if constexpr (HAS_MASK) {
        const int bh = a.blk_heads == 1 ? 0 : hg;
        blk_row = (const_u32 *)(a.blk + (((int64_t)b * a.blk_heads + bh) * a.row_blocks + rb) * a.blk_stride);
    }
    auto tile_code = [&](int t) -> int {
        if constexpr (HAS_MASK) {
            return (int)((blk_row[t >> 2] >> (8 * (t & 3))) & 0xffu);
        } else {
            return TILE_OPEN;
        }
    };
    const int kt_begin = split * a.tiles_per_split;
    const int kt_end = min(kt_begin + a.tiles_per_split, a.kv_tiles);
    auto next_tile = [&](int from) {
        int t = from;
        while (t < kt_end && tile_code(t) == TILE_SKIP) ++t;
        return t < kt_end ? t : kt_end;
    };

    // per-lane pieces of the transposing V read: row kb + j/4, logical chunk
    // 4*db + 2*(g&1) + (j&3)/2 (plus the slice), element 4*(j&1) inside the chunk
    const int g16 = lane >> 4, j16 = lane & 15;
    const int v_rsub = 4 * (g16 >> 1) + (j16 >> 2);
    const int v_lchunk0 = slice * (DS / 8) + 2 * (g16 & 1) + ((j16 & 3) >> 1);
    const int v_inner = 4 * (j16 & 1);

    int kt = next_tile(kt_begin);
    if (kt < kt_end) {
        issue_tile<D, NW, false>(k_lds, kbase, a.k_rs, kt * kTile, a.kv_len, wave, lane);
        issue_tile<D, NW, true>(v_lds, vbase, a.v_rs, kt * kTile, a.kv_len, wave, lane);
    }
    while (kt < kt_end) {
        const int code = tile_code(kt);
        const int nxt = next_tile(kt + 1);
        const int key0 = kt * kTile;
        const bool full_tile = key0 + kTile <= a.kv_len;

        wait_vm_barrier<NLD>();  // K(kt) is in LDS for every wave; V(kt) may still be landing

        // raw mask values of this lane's 32 keys (key0 + 32*blk2 + 8*q4 + 4*half + e); with two
        // slices only slice 0 adds the mask into its partial scores
        uint2 mraw[2][4];
        const bool use_mask = HAS_MASK && code == TILE_MASKED && slice == 0;
        if constexpr (HAS_MASK) {
            if (use_mask) {
                if (a.mask_vec && full_tile) {
#pragma unroll
                    for (int blk2 = 0; blk2 < 2; ++blk2)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            mraw[blk2][q4] = *reinterpret_cast<const uint2 *>(mrow + key0 + 32 * blk2 + 8 * q4 + 4 * half);
                } else {
                    // any alignment, any tail: element loads from clamped (in-bounds) keys
#pragma unroll
                    for (int blk2 = 0; blk2 < 2; ++blk2)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const int kf = key0 + 32 * blk2 + 8 * q4 + 4 * half;
                            uint16_t m16[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) m16[e] = mrow[min(kf + e, a.kv_len - 1)];
                            mraw[blk2][q4] = make_uint2(pack2(m16[0], m16[1]), pack2(m16[2], m16[3]));
                        }
                }
            }
        }

        // ---- S^T (64 keys x 32 queries) over this wave's head-dim slice
        float16v s[2];
#pragma unroll
        for (int blk2 = 0; blk2 < 2; ++blk2) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[blk2][r] = 0.f;
            const int krow = blk2 * 32 + col;
            const uint16_t *kr = &k_lds[krow * D];
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const int lch = slice * (DS / 8) + 2 * ks + half;
                const uint4v kf = *reinterpret_cast<const uint4v *>(kr + 8 * (lch ^ k_swz(krow)));
                s[blk2] = mfma32<BF16>(kf, qf[ks], s[blk2]);
                if constexpr (QSPLIT) s[blk2] = mfma32<BF16>(kf, qlo[ks], s[blk2]);
            }
        }

        // ---- scale and mask (consumed before the next K tile is requested, so waiting for the
        // mask loads never waits on that prefetch); this lane holds keys key0 + 32*blk2 + 8*(r/4) + 4*half + r%4
#pragma unroll
        for (int blk2 = 0; blk2 < 2; ++blk2)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float mvf = 0.f;
                    if (use_mask) {
                        const uint32_t word = e < 2 ? mraw[blk2][q4].x : mraw[blk2][q4].y;
                        const uint16_t m16 = (uint16_t)(word >> (16 * (e & 1)));
                        mvf = (a.mask_bf16 ? bf16_bits_to_f32(m16) : f16_bits_to_f32(m16)) * kLog2e;
                    }
                    s[blk2][4 * q4 + e] = fmaf(s[blk2][4 * q4 + e], a.score_scale, mvf);
                }
        if constexpr (NS > 1) {
#pragma unroll
            for (int blk2 = 0; blk2 < 2; ++blk2)
#pragma unroll
                for (int r = 0; r < 16; ++r) x_lds[((wave * 2 + blk2) * 16 + r) * 64 + lane] = s[blk2][r];
        }
        lds_done_barrier();  // every wave is done with K(kt) (and has posted its partial scores)
        if (nxt < kt_end) issue_tile<D, NW, false>(k_lds, kbase, a.k_rs, nxt * kTile, a.kv_len, wave, lane);
        if constexpr (NS > 1) {
            const int other = qwave * NS + (1 - slice);
#pragma unroll
            for (int blk2 = 0; blk2 < 2; ++blk2)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[blk2][r] += x_lds[((other * 2 + blk2) * 16 + r) * 64 + lane];
        }
        if (!full_tile) {
#pragma unroll
            for (int blk2 = 0; blk2 < 2; ++blk2)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (key0 + 32 * blk2 + 8 * (r >> 2) + 4 * half + (r & 3) >= a.kv_len) s[blk2][r] = -INFINITY;
        }

        // ---- online softmax for this lane's query (32 keys here, 32 in lane ^ 32)
        float mx = -INFINITY;
#pragma unroll
        for (int blk2 = 0; blk2 < 2; ++blk2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[blk2][r]);
        mx = max_with_other_half(mx);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float rowsum = 0.f;
        uint4v pb[4];  // B operands of O^T += V^T P^T: pb[2*blk2 + e] holds regs 8e..8e+7 of s[blk2]
#pragma unroll
        for (int blk2 = 0; blk2 < 2; ++blk2) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint16_t p16[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    p16[i] = to_kv16<BF16>(exp2f(s[blk2][8 * e + i] - m_use));
                    rowsum += from_kv16<BF16>(p16[i]);
                }
                pb[2 * blk2 + e] = uint4v{pack2(p16[0], p16[1]), pack2(p16[2], p16[3]), pack2(p16[4], p16[5]),
                                          pack2(p16[6], p16[7])};
            }
        }
        rowsum = sum_with_other_half(rowsum);
        l_run = l_run * alpha + rowsum;
        m_run = m_new;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_o[db][r] *= alpha;
        }

        // V(kt) landed for every wave (K(nxt) may still be in flight)
        if (nxt < kt_end) {
            wait_vm_barrier<NLD>();
        } else {
            wait_vm_barrier<0>();
        }

        // ---- O^T[d][query] += V^T[d][key] P^T[key][query]
        // A operand slot i of lane (m, half) is key 32*blk2 + 16*e + 8*(i/4) + 4*half + i%4, column m.
        // A 16-lane group g reads 4 keys x 16 columns per ds_read_b64_tr_b16: lane j of the
        // group points at row kb + j/4, columns c0 + 4*(j%4) .. +3; lane j receives
        // rows kb..kb+3 of column c0 + j.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int blk2 = u >> 1, e = u & 1;
            const int r0 = 32 * blk2 + 16 * e + v_rsub;      // rows r0 (slots 0..3) and r0 + 8 (slots 4..7)
            const uint16_t *vr0 = &v_lds[r0 * D + v_inner];
            const uint16_t *vr1 = &v_lds[(r0 + 8) * D + v_inner];
            const int sw0 = v_swz(r0), sw1 = v_swz(r0 + 8);
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const int lch = 4 * db + v_lchunk0;
                const short4v lo = read_tr16(vr0 + 8 * (lch ^ sw0));
                const short4v hi = read_tr16(vr1 + 8 * (lch ^ sw1));
                uint4v vf;
                vf[0] = pack2((uint16_t)lo[0], (uint16_t)lo[1]);
                vf[1] = pack2((uint16_t)lo[2], (uint16_t)lo[3]);
                vf[2] = pack2((uint16_t)hi[0], (uint16_t)hi[1]);
                vf[3] = pack2((uint16_t)hi[2], (uint16_t)hi[3]);
                acc_o[db] = mfma32<BF16>(vf, pb[u], acc_o[db]);
            }
        }
        lds_done_barrier();  // every wave is done with V(kt)
        if (nxt < kt_end) issue_tile<D, NW, true>(v_lds, vbase, a.v_rs, nxt * kTile, a.kv_len, wave, lane);
        kt = nxt;
    }

    // ---- epilogue: this lane holds O^T columns query `col`, rows d = slice*DS + 32*db + 8*(r/4) + 4*half + r%4
    if (!row_ok) return;
    if (a.splits == 1) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        float *orow = a.o + b * a.o_bs + (int64_t)row * a.o_rs + head * a.o_hs + slice * DS + 4 * half;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float4v x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc_o[db][4 * r4 + e] * inv;
                *reinterpret_cast<float4v *>(orow + 32 * db + 8 * r4) = x;
            }
    } else {
        const int64_t unit = (((int64_t)split * a.batch + b) * a.n_heads + head) * a.rows + row;
        float *prow = a.part + unit * D + slice * DS + 4 * half;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float4v x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc_o[db][4 * r4 + e];
                *reinterpret_cast<float4v *>(prow + 32 * db + 8 * r4) = x;
            }
        if (slice == 0 && half == 0) a.ml[unit] = make_float2(m_run, l_run);
    }
}

// One wave classifies one (query block, 64-key tile): TILE_SKIP when every
// entry is -inf, TILE_OPEN when every entry is zero, else TILE_MASKED.  Only
// entries of real rows (< rows) and keys (< kv_len) are read.  Grid:
// (ceil(kv_tiles / 4), row_blocks, batch * blk_heads), four waves per block.
__global__ __launch_bounds__(256) void classify_kernel(PrefillArgs a, uint8_t *blk) {
    const int lane = threadIdx.x & 63;
    const int kt = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (kt >= a.kv_tiles) return;
    const int rb = blockIdx.y;
    const int hg = blockIdx.z % a.blk_heads;
    const int b = blockIdx.z / a.blk_heads;
    const int slots = a.rows_per_wg * (a.blk_heads == 1 ? 1 : a.heads_per_wg);
    const int h0 = hg * a.heads_per_wg;
    const uint16_t *mbase = (const uint16_t *)a.mask + b * a.m_bs;
    const uint16_t neg_inf = a.mask_bf16 ? 0xFF80u : 0xFC00u;
    const int key0 = kt * kTile;
    bool any_visible = false, any_nonzero = false;
    if (a.mask_vec) {
        // 16 lanes per 64-key row, 4 keys (8 bytes) per lane, 4 rows per pass
        const int k4 = key0 + 4 * (lane & 15);
        for (int s = lane >> 4; s < slots; s += 4) {
            const int head = h0 + s / a.rows_per_wg;
            const int row = rb * a.rows_per_wg + s % a.rows_per_wg;
            if (row >= a.rows) continue;
            const uint16_t *mr = mbase + head * a.m_hs + (int64_t)row * a.m_rs;
            if (k4 + 4 <= a.kv_len) {
                const uint2 raw = *reinterpret_cast<const uint2 *>(mr + k4);
                const uint16_t m16[4] = {(uint16_t)(raw.x & 0xffffu), (uint16_t)(raw.x >> 16),
                                         (uint16_t)(raw.y & 0xffffu), (uint16_t)(raw.y >> 16)};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    any_visible |= m16[e] != neg_inf;
                    any_nonzero |= (m16[e] & 0x7fffu) != 0;
                }
            } else {
                for (int e = 0; e < 4; ++e) {
                    if (k4 + e < a.kv_len) {
                        const uint16_t m16 = mr[k4 + e];
                        any_visible |= m16 != neg_inf;
                        any_nonzero |= (m16 & 0x7fffu) != 0;
                    }
                }
            }
        }
    } else {
        const int key = key0 + lane;
        if (key < a.kv_len) {
            for (int s = 0; s < slots; ++s) {
                const int head = h0 + s / a.rows_per_wg;
                const int row = rb * a.rows_per_wg + s % a.rows_per_wg;
                if (row >= a.rows) continue;
                const uint16_t m16 = mbase[head * a.m_hs + (int64_t)row * a.m_rs + key];
                any_visible |= m16 != neg_inf;
                any_nonzero |= (m16 & 0x7fffu) != 0;
            }
        }
    }
    const bool vis = __ballot(any_visible) != 0;
    const bool nz = __ballot(any_nonzero) != 0;
    if (lane == 0) {
        uint8_t *out = blk + (((int64_t)b * a.blk_heads + hg) * a.row_blocks + rb) * a.blk_stride;
        out[kt] = !vis ? TILE_SKIP : (nz ? TILE_MASKED : TILE_OPEN);
    }
}

// Merge split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(PrefillArgs a) {
    constexpr int PER_UNIT = D / 4;
    const int64_t units = (int64_t)a.batch * a.n_heads * a.rows;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t unit = t / PER_UNIT;
    const int d4 = t % PER_UNIT;
    if (unit >= units) return;
    float mmax = -INFINITY;
    for (int s = 0; s < a.splits; ++s) mmax = fmaxf(mmax, a.ml[s * units + unit].x);
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
    if (mmax != -INFINITY) {
        for (int s = 0; s < a.splits; ++s) {
            const float2 ml = a.ml[s * units + unit];
            if (ml.x == -INFINITY) continue;
            const float w = exp2f(ml.x - mmax);
            l += w * ml.y;
            const float4v x = *reinterpret_cast<const float4v *>(a.part + (s * units + unit) * D + 4 * d4);
            acc += w * x;
        }
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int row = unit % a.rows;
    const int64_t bh = unit / a.rows;
    const int head = bh % a.n_heads;
    const int b = bh / a.n_heads;
    *reinterpret_cast<float4v *>(a.o + b * a.o_bs + (int64_t)row * a.o_rs + head * a.o_hs + 4 * d4) = acc * inv;
}

template <int D, int NW, bool BF16, bool HAS_MASK>
hipError_t launch_nw(const PrefillArgs &a, const PrefillPlan *plan, hipStream_t stream) {
    dim3 grid(plan->row_blocks, plan->head_groups, (unsigned)(a.batch * plan->splits));
    if constexpr (BF16) {
        if (!a.q_bf16) {
            hipLaunchKernelGGL((prefill_kernel<D, NW, true, HAS_MASK, true>), grid, dim3(64 * NW), 0, stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((prefill_kernel<D, NW, BF16, HAS_MASK, false>), grid, dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool BF16, bool HAS_MASK>
hipError_t launch_typed(const PrefillArgs &a, const PrefillPlan *plan, hipStream_t stream) {
    if (plan->waves == 4) return launch_nw<D, 4, BF16, HAS_MASK>(a, plan, stream);
    if constexpr (D <= 256) {
        if (plan->waves == 2) return launch_nw<D, 2, BF16, HAS_MASK>(a, plan, stream);
    }
    return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_combine(const PrefillArgs &a, hipStream_t stream) {
    const int64_t threads = (int64_t)a.batch * a.n_heads * a.rows * (D / 4);
    hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_for_dim(const PrefillArgs &a, const PrefillPlan *plan, bool bf16, hipStream_t stream) {
    const bool has_mask = a.mask != nullptr;
    hipError_t err;
    if (bf16) {
        err = has_mask ? launch_typed<D, true, true>(a, plan, stream) : launch_typed<D, true, false>(a, plan, stream);
    } else {
        err = has_mask ? launch_typed<D, false, true>(a, plan, stream) : launch_typed<D, false, false>(a, plan, stream);
    }
    if (err != hipSuccess) return err;
    if (plan->splits > 1) return launch_combine<D>(a, stream);
    return hipSuccess;
}

}  // namespace

static int pow2_at_least(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int plan_prefill(const attn_prefill_params *p, PrefillPlan *plan) {
    const int D = p->head_dim;
    plan->head_dim = D;
    plan->slices = D > 256 ? 2 : 1;
    plan->slice_dim = D / plan->slices;
    const int g = p->n_heads / p->n_kv_heads;
    // 4 waves hold 128 query slots (64 with two head-dim slices); at least 64 slots
    const int max_slots = plan->slices == 1 ? 128 : 64;
    int rpw = pow2_at_least(p->rows < 32 ? p->rows : 32);
    int hpw = 1;  // a power of two, so rows_per_wg * heads_per_wg can reach a multiple of 32
    for (int d = 1; d <= g; d *= 2)
        if (g % d == 0 && rpw * d <= max_slots) hpw = d;
    while ((rpw * hpw) % 64 != 0) rpw *= 2;
    while (rpw * hpw < max_slots && rpw < p->rows) rpw *= 2;
    plan->rows_per_wg = rpw;
    plan->heads_per_wg = hpw;
    plan->query_waves = rpw * hpw / 32;
    plan->waves = plan->query_waves * plan->slices;
    if (plan->waves != 4 && !(plan->waves == 2 && plan->slices == 1)) return ATTN_EINVAL;
    plan->row_blocks = (p->rows + rpw - 1) / rpw;
    plan->head_groups = p->n_heads / hpw;
    plan->kv_tiles = (p->kv_len + kTile - 1) / kTile;
    plan->blk_stride = (plan->kv_tiles + 3) & ~3;  // rows of tile codes are read as dwords
    const int64_t wgs = (int64_t)plan->row_blocks * plan->head_groups * p->batch;
    int splits = 1;
    if (wgs < 256 && plan->kv_tiles >= 4) {
        splits = (int)((512 + wgs - 1) / wgs);
        if (splits > plan->kv_tiles / 2) splits = plan->kv_tiles / 2;
        if (splits < 1) splits = 1;
    }
    plan->tiles_per_split = (plan->kv_tiles + splits - 1) / splits;
    plan->splits = plan->tiles_per_split > 0 ? (plan->kv_tiles + plan->tiles_per_split - 1) / plan->tiles_per_split : 1;
    if (plan->splits < 1) plan->splits = 1;
    size_t off = 0;
    if (p->mask_dtype != ATTN_NONE) {
        const int blk_heads = p->m_hs == 0 ? 1 : plan->head_groups;
        plan->blk_bytes = (size_t)p->batch * blk_heads * plan->row_blocks * plan->blk_stride;
    } else {
        plan->blk_bytes = 0;
    }
    plan->blk_offset = 0;
    off = align256(plan->blk_bytes);
    const size_t units = (size_t)p->batch * p->n_heads * p->rows;
    if (plan->splits > 1) {
        plan->ml_offset = off;
        plan->ml_bytes = (size_t)plan->splits * units * sizeof(float2);
        off = align256(off + plan->ml_bytes);
        plan->part_offset = off;
        plan->part_bytes = (size_t)plan->splits * units * D * sizeof(float);
        off = align256(off + plan->part_bytes);
    } else {
        plan->ml_offset = plan->ml_bytes = plan->part_offset = plan->part_bytes = 0;
    }
    plan->workspace_bytes = off;
    return ATTN_OK;
}

hipError_t launch_prefill(const attn_prefill_params *p, const PrefillPlan *plan, const void *q, const void *k,
                          const void *v, const void *mask, float *o, void *ws, hipStream_t stream) {
    PrefillArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.mask = p->mask_dtype == ATTN_NONE ? nullptr : mask;
    a.o = o;
    uint8_t *w = (uint8_t *)ws;
    a.blk = plan->blk_bytes ? w + plan->blk_offset : nullptr;
    a.ml = plan->splits > 1 ? (float2 *)(w + plan->ml_offset) : nullptr;
    a.part = plan->splits > 1 ? (float *)(w + plan->part_offset) : nullptr;
    a.q_bs = p->q_bs; a.q_rs = p->q_rs; a.q_hs = p->q_hs;
    a.k_bs = p->k_bs; a.k_rs = p->k_rs; a.k_hs = p->k_hs;
    a.v_bs = p->v_bs; a.v_rs = p->v_rs; a.v_hs = p->v_hs;
    a.m_bs = p->m_bs; a.m_hs = p->m_hs; a.m_rs = p->m_rs;
    a.o_bs = p->o_bs; a.o_rs = p->o_rs; a.o_hs = p->o_hs;
    a.batch = p->batch;
    a.rows = p->rows;
    a.kv_len = p->kv_len;
    a.n_heads = p->n_heads;
    a.group = p->n_heads / p->n_kv_heads;
    a.rows_per_wg = plan->rows_per_wg;
    a.heads_per_wg = plan->heads_per_wg;
    a.row_blocks = plan->row_blocks;
    a.head_groups = plan->head_groups;
    a.blk_heads = (p->mask_dtype != ATTN_NONE && p->m_hs != 0) ? plan->head_groups : 1;
    a.kv_tiles = plan->kv_tiles;
    a.blk_stride = plan->blk_stride;
    a.splits = plan->splits;
    a.tiles_per_split = plan->tiles_per_split;
    a.q_bf16 = p->q_dtype == ATTN_BF16;
    a.mask_bf16 = p->mask_dtype == ATTN_BF16;
    // 8-byte mask loads need every row start 8-byte aligned
    a.mask_vec = a.mask && (p->m_rs % 4 == 0) && (p->m_hs % 4 == 0) && (p->m_bs % 4 == 0) &&
                 (((uintptr_t)mask & 7u) == 0);
    a.score_scale = p->scale * kLog2e;

    if (a.mask) {
        dim3 grid((plan->kv_tiles + 3) / 4, plan->row_blocks, p->batch * a.blk_heads);
        hipLaunchKernelGGL(classify_kernel, grid, dim3(256), 0, stream, a, (uint8_t *)a.blk);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const bool bf16 = p->kv_dtype == ATTN_BF16;
    switch (plan->head_dim) {
    case 128: return launch_for_dim<128>(a, plan, bf16, stream);
    case 256: return launch_for_dim<256>(a, plan, bf16, stream);
    case 512: return launch_for_dim<512>(a, plan, bf16, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
