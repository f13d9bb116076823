// prefill_common.h -- what the prefill kernels (prefill.hip, narrow.hip) share:
// the kernel arguments, the constants of the online softmax, MFMA and packing
// helpers, and the LDS-DMA tile streams.  Not part of the public ABI.
#pragma once

#include <math.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "internal.h"

namespace attn {

struct PrefillArgs {
    const void *q, *k, *v, *mask;
    float *o;
    const uint8_t *blk;
    float *part;       // split partials (unnormalised O)
    float2 *ml;        // split partials (running max in log2 units, running sum)
    float *pair_part;  // paired row blocks: unnormalised O of each side [pairs][2][slots][D]
    float2 *pair_ml;   // paired row blocks: (m, l) of each side [pairs][2][slots]
    uint32_t *pair_cnt;  // paired row blocks: [pairs][arrivals, partial ready] (zeroed by the classify pass)
    uint32_t *status;    // status block: [0] error flags, [1] merged row blocks (zeroed at the start of every call)
    int64_t q_bs, q_rs, q_hs, k_bs, k_rs, k_hs, v_bs, v_rs, v_hs, m_bs, m_hs, m_rs, o_bs, o_rs, o_hs;
    int batch, rows, kv_len, n_heads, group;
    int rows_per_wg, heads_per_wg, row_blocks, head_groups, blk_heads;
    int kv_tiles, blk_stride, splits, tiles_per_split;
    int q_bf16, mask_bf16, mask_vec, mask_dma, pairing, n_pair_cnt;
    float score_scale;  // scale * log2(e)
};

// The eight-wave kernel for head_dim 128/256 (narrow.hip): launches it for the
// call's head dim, K/V type and mask type.
hipError_t launch_narrow_prefill(const PrefillArgs &a, const PrefillPlan *plan, bool bf16, hipStream_t stream);

namespace {

constexpr int kTile = 64;               // KV rows per step
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsAhead = 4;            // MFMA operand reads in flight ahead of their MFMA

// O and l are rescaled only when a row's running max grows by more than this
// many binary orders of magnitude; until then the stale max stays the
// reference, so P <= 2^8 (fine in f16, bf16 and the fp32 sums) and O / l is
// unchanged.  Rescales then happen a few times per row instead of per tile.
constexpr float kRescaleThreshold = 8.f;

// Words of the status block at the start of the workspace (ATTN_PREFILL_STATUS_BYTES).
constexpr int kStatusWords = ATTN_PREFILL_STATUS_BYTES / 4;
// Polls of a partner's ready flag before the wait gives up (each poll sleeps ~128 clocks).
constexpr int kPairWaitPolls = 1 << 22;


typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bhalf2v __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ float4v mfma16(uint4v a, uint4v b, float4v c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bhalf8, a), __builtin_bit_cast(bhalf8, b),
                                                       c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c,
                                                      0, 0, 0);
    }
}

// Max and sum over the four lanes l, l^16, l^32, l^48 (one column of a 16x16 tile)
__device__ __forceinline__ float max_over_rows(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return max_with_other_half(x);
}
__device__ __forceinline__ float sum_over_rows(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    return sum_with_other_half(x);
}

template <bool BF16>
__device__ __forceinline__ uint16_t to_kv16(float x) {
    if constexpr (BF16) {
        return f32_to_bf16_rne(x);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
}

// Two probabilities rounded to f16 (v_cvt_pk_f16_f32) and their exact sum as
// rounded (v_dot2 against (1, 1), fp32 accumulation), so that the rounding
// cancels in O / l.
__device__ __forceinline__ uint32_t pack_p_f16(float p0, float p1, float &sum) {
    const half2v v = {(_Float16)p0, (_Float16)p1};
    sum = __builtin_amdgcn_fdot2(v, half2v{(_Float16)1.f, (_Float16)1.f}, sum, false);
    return __builtin_bit_cast(uint32_t, v);
}

// Two probabilities as bf16 hi + lo pairs (about 16 significant bits; one bf16
// rounding, 2^-9 relative, breaks the error bound for a row that sees only a
// few keys), and their f32 sum.
__device__ __forceinline__ void pack_p_bf16(float p0, float p1, uint32_t &hi, uint32_t &lo, float &sum) {
    const bhalf2v h = {(__bf16)p0, (__bf16)p1};
    const bhalf2v l = {(__bf16)(p0 - (float)h[0]), (__bf16)(p1 - (float)h[1])};
    sum += p0 + p1;
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(4))) uint32_t const_u32;

// two consecutive ds_read_b64_tr_b16 results form one MFMA operand as read
__device__ __forceinline__ uint4v read_tr16_pair(const uint16_t *p0, const uint16_t *p1) {
    const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)p0));
    const uint2 hi = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)p1));
    return uint4v{lo.x, lo.y, hi.x, hi.y};
}

// LDS tile layouts (64 rows x D, no padding).  Chunk = 16 bytes = 8 elements.
//  K: logical chunk c of row r sits at physical chunk c ^ (r % 16); the S^T
//     A-operand read (16 consecutive rows, one chunk) hits 16 distinct banks.
//  V: logical chunk c of row r sits at physical chunk c ^ 4*(r % 4); the
//     transposing read (4 consecutive rows x 4 chunks per 32 lanes) hits 16
//     distinct bank groups.

// Row strides (elements) below this keep every offset inside a 64-row stage under 2^32 bytes.
constexpr int64_t kOff32Stride = (int64_t)1 << 25;

// One row of tile codes (a row block's byte per 64-key tile, padded to whole dwords),
// as the classify pass wrote it: its stages that are not skipped (SPT stages per tile
// code, the last tile possibly fewer), and the stage after the first `cut` of them.
// The whole wave scans the row, one dword (four codes) per lane, with a wave-wide sum
// or prefix sum; every lane gets the result.
template <int SPT>
struct CodeRow {
    const uint8_t *row;
    int stride, kv_tiles, n_stages;

    __device__ __forceinline__ int lane_stages(int w) const {  // unskipped stages in dword w
        int n = 0;
        if (w < stride / 4) {
            const uint32_t word = reinterpret_cast<const uint32_t *>(row)[w];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 4 * w + j;
                if (t < kv_tiles && ((word >> (8 * j)) & 0xffu) != TILE_SKIP) n += min(SPT, n_stages - t * SPT);
            }
        }
        return n;
    }
    __device__ __forceinline__ int count(int lane) const {
        int n = 0;
        for (int w0 = 0; w0 < stride / 4; w0 += 64) n += lane_stages(w0 + lane);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
        return __builtin_amdgcn_readfirstlane(n);
    }
    __device__ __forceinline__ int stage_after(int cut, int lane) const {
        int before = 0;  // unskipped stages in earlier passes
        for (int w0 = 0; w0 < stride / 4; w0 += 64) {
            const int w = w0 + lane;
            const int mine = lane_stages(w);
            int incl = mine;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int up = __shfl_up(incl, off);
                if (lane >= off) incl += up;
            }
            const uint64_t hit = __ballot(before + incl >= cut);
            if (hit) {
                const int L = __builtin_ctzll(hit);
                // in lane L: walk its four tiles from the count before it
                int n = before + incl - mine, at = n_stages;
                if (lane == L) {
                    const uint32_t word = reinterpret_cast<const uint32_t *>(row)[w];
                    for (int j = 0; j < 4; ++j) {
                        const int t = 4 * w + j;
                        if (t < kv_tiles && ((word >> (8 * j)) & 0xffu) != TILE_SKIP) {
                            const int k = min(SPT, n_stages - t * SPT);
                            if (n + k >= cut) {
                                at = t * SPT + (cut - n);
                                break;
                            }
                            n += k;
                        }
                    }
                }
                return __builtin_amdgcn_readfirstlane(__shfl(at, L));
            }
            before += __shfl(incl, 63);
        }
        return n_stages;
    }
};

// The tasks of workgroup (b, hg, idx): a row block and a stage range each.  Without
// pairing it is one row block (the last ones first: a causal frontier makes them the
// heaviest) over the workgroup's KV split.  With pairing, row blocks lo = p and
// hi = RB-1-p share two workgroups: side 0 takes the first half of their unskipped
// stages from hi, side 1 the rest of hi and then all of lo, so both sides carry the
// same load whatever the mask; when hi is cut, the side that finishes it second
// merges the two partial results (side0 says which side of a cut block task 0 is,
// -1 when it is not cut).
struct PrefillTasks {
    int rb0, beg0, end0, side0;
    int rb1, beg1, end1;
    int ntask, pair;
};
template <int SPT, bool HAS_MASK>
__device__ __forceinline__ PrefillTasks prefill_tasks(const PrefillArgs &a, int b, int hg, int idx, int split_begin,
                                                      int split_end, int n_stages, int lane) {
    PrefillTasks t{a.row_blocks - 1 - idx, split_begin, split_end, -1, 0, 0, 0, 1, 0};
    if constexpr (HAS_MASK) {
        if (a.pairing) {
            auto code_row = [&](int rbx) {
                const int bh = a.blk_heads == 1 ? 0 : hg;
                return CodeRow<SPT>{a.blk + (((int64_t)b * a.blk_heads + bh) * a.row_blocks + rbx) * a.blk_stride,
                                    a.blk_stride, a.kv_tiles, n_stages};
            };
            const int npairs = a.row_blocks >> 1;
            if (idx < 2 * npairs) {
                t.pair = idx >> 1;
                const int side = idx & 1;
                const int rb_lo = t.pair, rb_hi = a.row_blocks - 1 - t.pair;
                const int w_hi = code_row(rb_hi).count(lane);
                const int w_lo = code_row(rb_lo).count(lane);
                const int cut = min((w_hi + w_lo + 1) >> 1, w_hi);
                const bool shared = cut > 0 && cut < w_hi;
                const int s_cut = shared ? code_row(rb_hi).stage_after(cut, lane) : n_stages;
                t.beg0 = 0;
                t.end0 = n_stages;
                if (side == 0) {
                    t.rb0 = rb_hi;
                    t.end0 = s_cut;
                    t.side0 = shared ? 0 : -1;
                } else if (shared) {
                    t.rb0 = rb_hi;
                    t.beg0 = s_cut;
                    t.side0 = 1;
                    t.rb1 = rb_lo;
                    t.end1 = n_stages;
                    t.ntask = 2;
                } else {
                    t.rb0 = rb_lo;
                }
            } else {
                t.rb0 = npairs;  // the middle row block of an odd count
            }
        }
    }
    return t;
}

// The cut-pair protocol of the two workgroups that share a cut row block (pair unit pu):
// counters pair_cnt[2 pu] (arrivals) and pair_cnt[2 pu + 1] (partial ready), both zeroed
// by the classify pass.  The first side to arrive publishes its unnormalised partial O
// and (m, l) and raises the ready flag; the second side waits for the flag (bounded) and
// merges.  The two sides may run on different XCDs, whose L2 caches are not coherent with
// each other: the partials are written and read with agent-coherent (sc1) accesses and
// only the ready flag orders them, so no fence has to write back or invalidate an L2.
// `flag` is an LDS word every thread of the workgroup can read.

// True when this workgroup arrives second (it merges), false when first (it publishes).
__device__ __forceinline__ bool pair_arrive(const PrefillArgs &a, int64_t pu, int *flag) {
    if (threadIdx.x == 0)
        *flag = (int)__hip_atomic_fetch_add(a.pair_cnt + 2 * pu, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return *flag != 0;
}
// The publishing side's (m, l) of one query slot.
__device__ __forceinline__ void pair_store_ml(const PrefillArgs &a, int64_t pu, int side, int slot, float m, float l) {
    const int slots = a.rows_per_wg * a.heads_per_wg;
    __hip_atomic_store(&a.pair_ml[(pu * 2 + side) * slots + slot].x, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&a.pair_ml[(pu * 2 + side) * slots + slot].y, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// After every wave's partial stores: once they have all completed, raise the ready flag.
__device__ __forceinline__ void pair_ready(const PrefillArgs &a, int64_t pu) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's partial is out
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(a.pair_cnt + 2 * pu + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The merging side waits for the ready flag, at most kPairWaitPolls polls, so that no wave
// can wait forever.  Returns true when it gave up: the partner's partial is then not used,
// the row block is written as NaN and the status block records the expiry.  A completed
// wait counts one merged row block in the status block.
__device__ __forceinline__ bool pair_wait(const PrefillArgs &a, int64_t pu, int *flag) {
    if (threadIdx.x == 0) {
        bool seen = false;
        for (int spin = 0; spin < kPairWaitPolls; ++spin) {
            if (__hip_atomic_load(a.pair_cnt + 2 * pu + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                seen = true;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (seen) {
            __hip_atomic_fetch_add(a.status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            __hip_atomic_fetch_or(a.status, (uint32_t)ATTN_PREFILL_WAIT_EXPIRED, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        }
        *flag = seen ? 1 : 2;
    }
    __syncthreads();
    return *flag == 2;
}
// The other side's (m, l) of one query slot (complete before its ready flag, which the
// caller has observed).
__device__ __forceinline__ float2 pair_load_ml(const PrefillArgs &a, int64_t pu, int other, int slot) {
    const int slots = a.rows_per_wg * a.heads_per_wg;
    return make_float2(
        __hip_atomic_load(&a.pair_ml[(pu * 2 + other) * slots + slot].x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
        __hip_atomic_load(&a.pair_ml[(pu * 2 + other) * slots + slot].y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Raw buffer descriptors (word 3 of the resource) and the cache policy that makes a
// buffer access coherent at agent scope (sc1).
constexpr int kRawBufferFlags = 0x00020000;
constexpr int kAgentCoherent = 16;

constexpr int cgcd(int x, int y) { return y == 0 ? x : cgcd(y, x % y); }

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// A wave-uniform pointer, made visibly uniform so that it can live in SGPRs.
__device__ __forceinline__ const char *uniform_ptr(const char *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const char *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Streams BK-row stages of K or V into LDS with global_load_lds_dwordx4: a
// wave-instruction fills 64 consecutive 16-byte LDS slots starting at M0, so
// each lane fetches the global chunk that belongs in its slot.  Instruction
// `it` of wave w covers rows row0 = (it*NW + w)*RPI .. +RPI-1; a lane's row
// within them (lrow) is fixed and its swizzled chunk repeats with a short
// period in `it`, so the lane offsets are computed once and each instruction
// only needs a scalar row base (no vector arithmetic per load).  Rows past
// kv_len (last stage only) fetch row kv_len-1: finite data whose keys are
// masked to -inf.
//
// SWZ is the chunk swizzle of the LDS layout: chunk c of row r is stored at
// c ^ f(r), with f(r) = r & 15 (K), 4*(r & 3) (V read by 32x32 MFMA tiles) or
// 2*(r & 7) (V read by 16x16 MFMA tiles); each keeps its tile's operand reads
// free of bank conflicts.
//
// The loads are issued from inline asm so the compiler does not treat every
// later LDS read as dependent on them (its conservative vmcnt(0) would drain
// the prefetch of the next stage); the explicit waits in the kernel cover
// them.  M0 is a reserved register that inline asm may not declare
// clobbered; nothing else in these kernels reads it (no movrel, sendmsg or
// LDS-DMA intrinsic), so writing it here is safe.
constexpr int kSwzK = 0, kSwzV32 = 1, kSwzV16 = 2;
template <int D, int NW, int BK, int SWZ>
struct TileStream {
    static constexpr int CH = D / 8;
    static constexpr int RPI = 64 / CH;                  // rows per instruction
    static constexpr int GR = NW * RPI;                  // rows one instruction of every wave covers
    static constexpr int NLD = BK / GR;                  // instructions per wave per stage
    // the swizzle term of instruction `it` repeats with period P in `it`
    static constexpr int PERIOD_ROWS = SWZ == kSwzV32 ? 4 : SWZ == kSwzV16 ? 8 : 16;
    static constexpr int P = PERIOD_ROWS / cgcd(PERIOD_ROWS, GR) < NLD ? PERIOD_ROWS / cgcd(PERIOD_ROWS, GR) : NLD;
    int lrow, inv;
    uint32_t voff[P];   // byte offset of this lane's 16 bytes from the instruction's first row

    __device__ __forceinline__ void init(int lane, int wave, int64_t row_stride) {
        lrow = lane / CH;
        const int lch = lane % CH;
        inv = lch ^ uniform_swz(lrow);
#pragma unroll
        for (int r = 0; r < P; ++r)
            voff[r] = (uint32_t)((lrow * row_stride + 8 * (inv ^ uniform_swz((r * NW + wave) * RPI))) * 2);
    }
    // f(r); for a row r = row0 + lrow with row0 a multiple of RPI and lrow < RPI,
    // f(r) = f(row0) ^ f(lrow)
    __device__ __forceinline__ static int uniform_swz(int row0) {
        return SWZ == kSwzV32 ? 4 * (row0 & 3) : SWZ == kSwzV16 ? 2 * (row0 & 7) : (row0 & 15);
    }

    // A stage of BK rows that all exist: one scalar base per stage and a 32-bit
    // lane offset per instruction (the row stride times BK rows fits in 32 bits,
    // which the caller checks).
    __device__ __forceinline__ void issue_full(uint16_t *lds, const uint16_t *base, int64_t row_stride, int key0,
                                               int wave) const {
        const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void *)lds;
        const char *stage = uniform_ptr((const char *)(base + (int64_t)(key0 + wave * RPI) * row_stride));
        const uint32_t step = (uint32_t)(GR * row_stride * 2);
#pragma unroll
        for (int it = 0; it < NLD; ++it) {
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base + (it * NW + wave) * 1024);
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff[it % P] + it * step),
                         "s"(stage)
                         : "memory");
        }
    }
    // The ragged last stage: rows past kv_len fetch row kv_len-1 instead.
    __device__ __forceinline__ void issue_tail(uint16_t *lds, const uint16_t *base, int64_t row_stride, int key0,
                                               int kv_len, int wave) const {
        const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void *)lds;
#pragma unroll 1
        for (int it = 0; it < NLD; ++it) {
            const int row0 = (it * NW + wave) * RPI;
            const int ch = inv ^ uniform_swz(row0);
            int grow = key0 + row0 + lrow;
            grow = grow < kv_len ? grow : kv_len - 1;
            const uint16_t *src = base + (int64_t)grow * row_stride + ch * 8;
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base + (it * NW + wave) * 1024);
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory");
        }
    }
    __device__ __forceinline__ void issue(uint16_t *lds, const uint16_t *base, int64_t row_stride, int key0,
                                          int kv_len, int wave, bool full) const {
        if (full && row_stride < kOff32Stride) issue_full(lds, base, row_stride, key0, wave);
        else issue_tail(lds, base, row_stride, key0, kv_len, wave);
    }
    // A full stage one instruction at a time, so that its loads can be spread between
    // other work: stage_ptr once per stage, then issue_one for it = 0 .. NLD-1 (it a
    // compile-time constant).
    __device__ __forceinline__ static const char *stage_ptr(const uint16_t *base, int64_t row_stride, int key0,
                                                            int wave) {
        return uniform_ptr((const char *)(base + (int64_t)(key0 + wave * RPI) * row_stride));
    }
    __device__ __forceinline__ void issue_one(uint16_t *lds, const char *stage, int64_t row_stride, int it,
                                              int wave) const {
        const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void *)lds;
        const uint32_t step = (uint32_t)(GR * row_stride * 2);
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base + (it * NW + wave) * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff[it % P] + it * step),
                     "s"(stage)
                     : "memory");
    }
};

// S^T accumulation kept in VGPRs.  A kernel that holds O in AGPRs gets AGPR accumulators
// for every MFMA the compiler emits, so an S accumulator there would evict an O block to
// VGPRs and back on every stage.  Written out, the chain's accumulator stays in VGPRs
// (dst = srcC, which back-to-back MFMAs of one opcode accumulate without wait states).  The
// compiler cannot see these MFMAs for its hazard checks: s_wait_after_mfma_vgpr() must
// separate the last of them from any other read of the accumulator.
__device__ __forceinline__ void mfma_f16_vacc_first(float16v &d, const uint4v &a, const uint4v &b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_f16_vacc(float16v &d, const uint4v &a, const uint4v &b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_bf16_vacc_first(float16v &d, const uint4v &a, const uint4v &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_bf16_vacc(float16v &d, const uint4v &a, const uint4v &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// 16 wait states: more than an 8-pass XDL result needs before a VALU, LDS or memory read of it.
__device__ __forceinline__ void s_wait_after_mfma_vgpr(float16v &d) {
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(d));
}

// x *= f for an accumulator element that lives in an AGPR.  Written out so that
// the only vector-ALU access to the O accumulator is this rare rescale: the
// compiler then keeps the accumulator in AGPRs next to the MFMAs instead of
// copying it to VGPRs on every stage.
__device__ __forceinline__ float scale_acc(float x, float f) {
    float t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(x), "=&v"(t)
                 : "v"(f));
    return x;
}

// Wait until every vector-memory operation and every LDS read of this wave has
// completed, then meet the other waves.  At the start of a stage this is the one
// barrier of the stage: once every wave is past it, no wave reads the previous
// stage's buffers any more, so the next stage may be requested into them.
__device__ __forceinline__ void wait_all_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void lds_done_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace
}  // namespace attn
