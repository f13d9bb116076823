// decode.hip -- single-query attention over a paged KV cache on gfx950.
//
// What is computed follows ferrum-kernels 0.8.3,
// src/backend/metal/vnext_ops/causal_attention.rs (the attention dispatch
// over fixed-size KV pages read through a per-sequence page table; query head
// h reads KV head h / (query_heads / key_value_heads); the context includes
// the token the step wrote).
//
// Design: decode is bound by HBM reads of K and V; the kernel keeps enough
// bytes in flight and keeps the arithmetic off the vector ALUs.
//  * Split-KV on a balanced line: every (sequence, KV head group) unit owns
//    ceil(context / 32) tiles of 32 tokens; the units are laid end to end and
//    range g is tiles [g*per, (g+1)*per) of that line (cut at unit
//    boundaries), so every range streams the same number of K/V bytes.  The
//    grid is the workgroups the chip runs at once; per is set on the device so
//    the ranges fill the fewest whole rounds of that grid, and workgroup w
//    takes ranges w, w + grid, ...  Each K/V row is read once for all query
//    heads of its KV head; a second kernel merges the pieces with a
//    log-sum-exp reduction.
//  * The (up to 16) query heads of a KV head are the 16 columns of a
//    v_mfma_f32_16x16x32 tile: S^T = K Q^T and O^T = V^T P^T run on the
//    matrix cores; P^T goes from the S^T accumulators straight into the
//    B operand, and V^T fragments come from ds_read_b64_tr_b16.
//  * Each wave streams its own 32-token K and V tiles into a private,
//    double-buffered LDS region with global_load_lds_dwordx4 (the next tile
//    is in flight while the current one is used), XOR-swizzled so the MFMA
//    operand reads are free of bank conflicts.  The chunk's page ids are
//    read once into LDS.
//  * The waves' states are merged in LDS at the end of the chunk.
#include <math.h>

#include <atomic>

#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTok = 32;      // tokens per wave step
// the (sequence, KV head group) units are laid end to end as 32-token tiles and
// every range takes between this many and (page sizes of 4 tokens and more) four times
// as many of them
constexpr int kDecodeMinTilesPerRange = 32;
constexpr int kDecodeMaxTilesPerRange = 128;
// page ids of one piece: a piece of kDecodeMinTilesPerRange tiles at page size 1, and of
// up to 32 * page_size tiles at larger page sizes
constexpr int kPgCap = kDecodeMinTilesPerRange * kTok + 2;
constexpr int kDecodeFallbackSlots = 512;  // without a device query

struct DecodeArgs {
    const float *q;
    const uint16_t *k_pool, *v_pool;
    const int32_t *page_table, *context_lens;
    float *o;
    float *part;
    float2 *ml;
    int64_t q_bs, q_hs, o_bs, o_hs, page_stride, token_stride, head_stride;
    int batch, n_heads, group, heads_per_wg, page_size, page_shift, max_pages, num_pages, ctx_cap;
    int hgroups;     // workgroup head groups per sequence
    int per_min, per_max;  // tiles (of kTok tokens) per range
    int slots;       // workgroups the chip runs at once (the grid)
    int max_splits;  // pieces per unit at most
    float score_scale;
};

typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

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

// (x[l], x[l ^ 16]) and (x[l], x[l ^ 32]) pairs; max and sum of a pair are symmetric
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

__device__ __forceinline__ int clamp_ctx(int c, int cap) { return c < 0 ? 0 : (c > cap ? cap : c); }

__device__ __forceinline__ int seq_tiles(const DecodeArgs &a, int b) {
    return (clamp_ctx(a.context_lens[b], a.ctx_cap) + kTok - 1) / kTok;
}

// Position of sequence b on the tile line.  Wave-wide: 64 sequences per step,
// an inclusive scan of their tile counts across the lanes.
struct SeqLoc {
    int b, tiles;    // sequence and its tiles per unit
    int64_t start;   // first tile of the sequence's units on the line
};

__device__ __forceinline__ int64_t scan_lanes(int64_t x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// The sequence whose units hold line tile `pos`, searching from sequence b0 whose
// units start at `base`; false when pos is past the end of the line.
__device__ bool locate_tile(const DecodeArgs &a, int64_t pos, int b0, int64_t base, SeqLoc &out) {
    const int lane = threadIdx.x & 63;
    for (; b0 < a.batch; b0 += 64) {
        const int bb = b0 + lane;
        const int t = bb < a.batch ? seq_tiles(a, bb) : 0;
        const int64_t incl = scan_lanes((int64_t)t * a.hgroups, lane);
        const int64_t total = __shfl(incl, 63);
        if (pos < base + total) {
            const int l = __builtin_ctzll(__ballot(base + incl > pos));
            out.b = b0 + l;
            out.tiles = __shfl(t, l);
            out.start = base + __shfl(incl, l) - (int64_t)out.tiles * a.hgroups;
            return true;
        }
        base += total;
    }
    return false;
}

// Tiles per range for a line of `total` tiles: the ranges fill the fewest whole rounds of
// `slots` workgroups at no more than per_max tiles each, and hold at least per_min.
__device__ __forceinline__ int per_for_line(const DecodeArgs &a, int64_t total) {
    const int64_t cap = (int64_t)a.slots * a.per_max;
    const int64_t rounds = total > cap ? (total + cap - 1) / cap : 1;
    const int64_t per = (total + rounds * a.slots - 1) / (rounds * a.slots);
    return (int)(per < a.per_min ? a.per_min : per);
}

// The line's length in tiles (wave-wide).
__device__ int64_t line_tiles(const DecodeArgs &a) {
    const int lane = threadIdx.x & 63;
    int64_t total = 0;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
        const int bb = b0 + lane;
        const int64_t t = bb < a.batch ? (int64_t)seq_tiles(a, bb) * a.hgroups : 0;
        total += __shfl(scan_lanes(t, lane), 63);
    }
    return total;
}

__device__ __forceinline__ int page_of(const DecodeArgs &a, int t) {
    return a.page_shift >= 0 ? (t >> a.page_shift) : t / a.page_size;
}

// LDS tile layouts (32 token rows x D, chunks of 16 bytes):
//  K: logical chunk c of row r at physical c ^ (r % 16)   (A-operand reads: 16 rows, one chunk)
//  V: logical chunk c of row r at physical c ^ 2*(r % 8)   (transposing reads: 8 rows x 2 chunks)
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return (row & 7) << 1; }

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Stream the K and V rows of tokens base..base+31 (clamped to t1-1) into one
// LDS buffer pair of this wave.  Each global_load_lds_dwordx4 fills 64
// consecutive 16-byte slots from M0; every call issues exactly 2*NLD of them.
// Issued from inline asm so the compiler's own waits do not drain it (see
// the explicit vmcnt waits in the kernel).  M0 is read only by these loads.
// The loads are nontemporal (nt): every K/V row is read once per call and the
// pool is far larger than the last-level cache, and streaming reads with the
// hint run about 15% faster than plain ones on this GPU.
template <int D>
__device__ __forceinline__ void issue_kv(const DecodeArgs &a, uint16_t *k_tile, uint16_t *v_tile, const int *s_pg,
                                        int pg0, int base, int t1, int64_t head_off, int lane) {
    constexpr int CH = D / 8;
    constexpr int NLD = kTok * CH / 64;
    int64_t row_off[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int row = (i * 64 + lane) / CH;
        int t = base + row;
        t = t < t1 ? t : t1 - 1;
        const int pg = page_of(a, t);
        const int page = s_pg[pg - pg0];
        row_off[i] = (int64_t)page * a.page_stride + (int64_t)(t - pg * a.page_size) * a.token_stride + head_off;
    }
    const uint32_t kb = (uint32_t)(uintptr_t)(lds_void *)k_tile;
    const uint32_t vb = (uint32_t)(uintptr_t)(lds_void *)v_tile;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int slot = i * 64 + lane;
        const int row = slot / CH, pch = slot % CH;
        const uint16_t *ksrc = a.k_pool + row_off[i] + 8 * (pch ^ k_swz(row));
        const uint16_t *vsrc = a.v_pool + row_off[i] + 8 * (pch ^ v_swz(row));
        const uint32_t mk = __builtin_amdgcn_readfirstlane(kb + i * 1024);
        const uint32_t mv = __builtin_amdgcn_readfirstlane(vb + i * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(mk), "v"(ksrc) : "memory");
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(mv), "v"(vsrc) : "memory");
    }
}

// One piece: tokens [t0, t1) of sequence b for workgroup head group hg, written
// as partial `split` of its units.
template <int D, int NWD, bool BF16>
__device__ __forceinline__ void decode_piece(const DecodeArgs &a, uint16_t *kv_lds, int *s_pg, int b, int hg, int t0,
                                             int t1, int split) {
    constexpr int CH = D / 8;
    constexpr int TILE = kTok * D;             // elements of one 32-token tile
    constexpr int NLD = kTok * CH / 64;        // load instructions per tile per wave
    constexpr int KSTEPS = D / 32;             // MFMA k-steps of S^T
    constexpr int DBLK = D / 16;               // 16-row blocks of O^T

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int hsplit = a.group / a.heads_per_wg;
    const int kvh = hg / hsplit;
    const int head0 = kvh * a.group + (hg % hsplit) * a.heads_per_wg;
    const int64_t unit0 = (int64_t)b * a.n_heads + head0;

    // page ids of this piece (entries past the context are never read)
    const int pg0 = page_of(a, t0);
    const int npg = page_of(a, t1 - 1) - pg0 + 1;
    for (int i = threadIdx.x; i < npg; i += blockDim.x) {
        int page = a.page_table[(int64_t)b * a.max_pages + pg0 + i];
        s_pg[i] = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    }
    __syncthreads();

    // Q^T as the B operand of S^T = K Q^T: column = query slot (lane % 16), k = 32*ks + 8*(lane/16) + i
    const int slot = lane & 15, g4 = lane >> 4;
    const bool slot_ok = slot < a.heads_per_wg;
    uint4v qf[KSTEPS];
    uint4v qlo[BF16 ? KSTEPS : 1];
    {
        const float *qp = a.q + b * a.q_bs + (int64_t)(head0 + (slot_ok ? slot : 0)) * a.q_hs + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const float4v x0 = *reinterpret_cast<const float4v *>(qp + 32 * ks);
            const float4v x1 = *reinterpret_cast<const float4v *>(qp + 32 * ks + 4);
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = slot_ok ? x0[e] * a.score_scale : 0.f;
                x[4 + e] = slot_ok ? x1[e] * a.score_scale : 0.f;
            }
            uint16_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = to_kv16<BF16>(x[e]);
            qf[ks] = uint4v{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
            if constexpr (BF16) {
                // bf16 keeps 8 significant bits: carry the rest of Q in a second operand
                uint16_t r[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = f32_to_bf16_rne(x[e] - bf16_bits_to_f32(h[e]));
                qlo[ks] = uint4v{pack2(r[0], r[1]), pack2(r[2], r[3]), pack2(r[4], r[5]), pack2(r[6], r[7])};
            }
        }
    }

    float4v acc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) acc[db] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    uint16_t *wbase = kv_lds + wave * 4 * TILE;
    const int64_t head_off = (int64_t)kvh * a.head_stride;
    // per-lane pieces of the transposing V read: row kb + j/4, logical chunk 2*db + (j&3)/2, element 4*(j&1)
    const int v_rsub = lane & 15;
    int base = t0 + kTok * wave;
    int buf = 0;
    if (base < t1) issue_kv<D>(a, wbase, wbase + TILE, s_pg, pg0, base, t1, head_off, lane);
    while (base < t1) {
        const int nbase = base + kTok * NWD;
        const bool has_next = nbase < t1;
        if (has_next) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the other buffer's reads are done
            uint16_t *nb = wbase + (buf ^ 1) * 2 * TILE;
            issue_kv<D>(a, nb, nb + TILE, s_pg, pg0, nbase, t1, head_off, lane);
            wait_vm<2 * NLD>();
        } else {
            wait_vm<0>();
        }
        const uint16_t *k_tile = wbase + buf * 2 * TILE;
        const uint16_t *v_tile = k_tile + TILE;

        // ---- S^T (32 tokens x 16 slots): lane holds slot `slot`, tokens 16*blk + 4*g4 + r
        float4v s[2];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            s[blk] = float4v{0.f, 0.f, 0.f, 0.f};
            const int row = 16 * blk + (lane & 15);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const uint4v kf = *reinterpret_cast<const uint4v *>(k_tile + row * D + 8 * ((4 * ks + g4) ^ k_swz(row)));
                s[blk] = mfma16<BF16>(kf, qf[ks], s[blk]);
                if constexpr (BF16) s[blk] = mfma16<BF16>(kf, qlo[ks], s[blk]);
            }
        }
        if (base + kTok > t1) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (base + 16 * blk + 4 * g4 + r >= t1) s[blk][r] = -INFINITY;
        }

        // ---- online softmax per slot (8 tokens here, the other 24 in lanes ^16, ^32, ^48)
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[blk][r]);
        mx = max_over_rows(mx);
        const float m_new = fmaxf(m_run, mx);   // finite: token `base` is real
        const float alpha = exp2f(m_run - m_new);
        uint16_t p16[8];
        float ps = 0.f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p16[4 * blk + r] = to_kv16<BF16>(exp2f(s[blk][r] - m_new));
                ps += from_kv16<BF16>(p16[4 * blk + r]);
            }
        ps = sum_over_rows(ps);
        l_run = l_run * alpha + ps;
        m_run = m_new;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db) acc[db] *= alpha;
        }
        // P^T as the B operand: k slot i <-> token 4*g4 + i (i < 4) and 16 + 4*g4 + (i - 4)
        const uint4v pb = uint4v{pack2(p16[0], p16[1]), pack2(p16[2], p16[3]), pack2(p16[4], p16[5]),
                                 pack2(p16[6], p16[7])};

        // ---- O^T[d][slot] += V^T[d][token] P^T[token][slot]
        // A operand: row d = 16*db + lane%16, k slots as above.  A 16-lane group reads rows kb..kb+3
        // (kb = 4*g4, then 16 + 4*g4) x 16 columns per ds_read_b64_tr_b16: lane j points at row
        // kb + j/4, columns 16*db + 4*(j%4), and receives rows kb..kb+3 of column 16*db + j.
        {
            const int r0 = 4 * g4 + (v_rsub >> 2), r1 = r0 + 16;
            const uint16_t *v0 = v_tile + r0 * D + 4 * (v_rsub & 1);
            const uint16_t *v1 = v_tile + r1 * D + 4 * (v_rsub & 1);
            const int c0 = (v_rsub & 3) >> 1;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) {
                const int lch = 2 * db + c0;
                const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(v0 + 8 * (lch ^ v_swz(r0))));
                const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(v1 + 8 * (lch ^ v_swz(r1))));
                const uint4v vf = uint4v{pack2((uint16_t)lo[0], (uint16_t)lo[1]), pack2((uint16_t)lo[2], (uint16_t)lo[3]),
                                         pack2((uint16_t)hi[0], (uint16_t)hi[1]), pack2((uint16_t)hi[2], (uint16_t)hi[3])};
                acc[db] = mfma16<BF16>(vf, pb, acc[db]);
            }
        }
        base = nbase;
        buf ^= 1;
    }

    // ---- merge the waves through LDS (the tiles are no longer needed)
    __syncthreads();
    float *s_o = reinterpret_cast<float *>(kv_lds);              // [wave][slot][D]
    float2 *s_ml = reinterpret_cast<float2 *>(s_o + NWD * 16 * D);  // [wave][slot]
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
        *reinterpret_cast<float4v *>(s_o + (wave * 16 + slot) * D + 16 * db + 4 * g4) = acc[db];
    if (g4 == 0) s_ml[wave * 16 + slot] = make_float2(m_run, l_run);
    __syncthreads();
    for (int e = threadIdx.x; e < a.heads_per_wg * D; e += blockDim.x) {
        const int sl = e / D, d = e % D;
        float mmax = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWD; ++w) mmax = fmaxf(mmax, s_ml[w * 16 + sl].x);
        float accv = 0.f, lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NWD; ++w) {
            const float2 ml = s_ml[w * 16 + sl];
            if (ml.x == -INFINITY) continue;  // this wave walked no token
            const float wgt = exp2f(ml.x - mmax);
            accv = fmaf(wgt, s_o[(w * 16 + sl) * D + d], accv);
            lsum = fmaf(wgt, ml.y, lsum);
        }
        const int64_t u = (unit0 + sl) * a.max_splits + split;
        a.part[u * D + d] = accv;
        if (d == 0) a.ml[u] = make_float2(mmax, lsum);
    }
    __syncthreads();  // the next piece reuses the tiles and page ids
}

template <int D, int NWD, bool BF16>
__global__ __launch_bounds__(64 * NWD) void decode_partial_kernel(DecodeArgs a) {
    constexpr int TILE = kTok * D;
    __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[NWD * 4 * TILE];   // [wave][buffer][K, V]
    __shared__ int s_pg[kPgCap];

    const int64_t total = line_tiles(a);
    const int per = per_for_line(a, total);
    // ranges g = blockIdx.x, blockIdx.x + gridDim.x, ...: line tiles [r0, r1), cut at unit
    // boundaries into pieces
    for (int64_t g = blockIdx.x; g * per < total; g += gridDim.x) {
        const int64_t r0 = g * per, r1 = r0 + per;
        SeqLoc loc;
        if (!locate_tile(a, r0, 0, 0, loc)) break;
        int64_t pos = r0;
        for (;;) {
            const int hg = (int)((pos - loc.start) / loc.tiles);
            const int64_t u0 = loc.start + (int64_t)hg * loc.tiles, u1 = u0 + loc.tiles;
            const int64_t e = u1 < r1 ? u1 : r1;
            const int ctx = clamp_ctx(a.context_lens[loc.b], a.ctx_cap);
            const int t0 = (int)(pos - u0) * kTok;
            const int t1 = min((int)(e - u0) * kTok, ctx);
            decode_piece<D, NWD, BF16>(a, kv_lds, s_pg, loc.b, hg, t0, t1, (int)(g - u0 / per));
            pos = e;
            if (pos >= r1) break;
            const int64_t seq_end = loc.start + (int64_t)loc.tiles * a.hgroups;
            if (pos >= seq_end && !locate_tile(a, pos, loc.b + 1, seq_end, loc)) break;
        }
    }
}

// One wave per (sequence, query head): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// over the pieces of its unit.
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
    constexpr int PER_LANE = D / 64;
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= (int64_t)a.batch * a.n_heads) return;
    const int b = unit / a.n_heads, head = unit % a.n_heads;
    // one pass over the lengths: the line's length (hence the tiles per range) and the
    // start of sequence b's units
    int64_t total = 0, start = 0;
    int tiles = 0;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
        const int bb = b0 + lane;
        const int tb = bb < a.batch ? seq_tiles(a, bb) : 0;
        const int64_t t = (int64_t)tb * a.hgroups;
        const int64_t incl = scan_lanes(t, lane);
        if (b >= b0 && b < b0 + 64) {
            start = total + __shfl(incl - t, b - b0);
            tiles = __shfl(tb, b - b0);
        }
        total += __shfl(incl, 63);
    }
    const int per = per_for_line(a, total);
    const int64_t u0 = start + (int64_t)(head / a.heads_per_wg) * tiles;
    int nsplit = tiles == 0 ? 0 : (int)((u0 + tiles - 1) / per - u0 / per + 1);
    if (nsplit > a.max_splits) nsplit = a.max_splits;
    float o[PER_LANE], lsum;
    merge_pieces<D>(a.ml + unit * a.max_splits, a.part + unit * a.max_splits * D, nsplit, lane, o, lsum);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float *orow = a.o + b * a.o_bs + (int64_t)head * a.o_hs + lane * PER_LANE;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) orow[i] = o[i] * inv;
}

// Workgroups of decode_partial_kernel<D, 1, BF16> the current device runs at once,
// looked up once per (device, kernel); CUs x 2 if the runtime cannot say.
template <int D, bool BF16>
int decode_slots_typed() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices] = {};
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kDecodeFallbackSlots;
    if (dev < kMaxDevices && cache[dev].load() > 0) return cache[dev].load();
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return kDecodeFallbackSlots;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(
                                                                   &decode_partial_kernel<D, 1, BF16>),
                                                     64, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 2;
    const int slots = cus * per_cu;
    if (dev < kMaxDevices) cache[dev].store(slots);
    return slots;
}

template <int D, bool BF16>
hipError_t launch_typed(const DecodeArgs &a, int64_t grid, hipStream_t stream) {
    // one wave per workgroup: 32 KiB (d 128) / 64 KiB (d 256) of double-buffered tiles, so several
    // workgroups share a CU and one's first-tile latency overlaps another's steady state
    constexpr int NWD = 1;
    hipLaunchKernelGGL((decode_partial_kernel<D, NWD, BF16>), dim3((unsigned)grid), dim3(64 * NWD), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t units = (int64_t)a.batch * a.n_heads;
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

int decode_slots(int head_dim, bool bf16) {
    switch (head_dim) {
    case 128: return bf16 ? decode_slots_typed<128, true>() : decode_slots_typed<128, false>();
    case 256: return bf16 ? decode_slots_typed<256, true>() : decode_slots_typed<256, false>();
    default: return kDecodeFallbackSlots;
    }
}

}  // namespace

int plan_decode(const attn_decode_params *p, DecodePlan *plan) {
    plan->head_dim = p->head_dim;
    plan->group = p->n_heads / p->n_kv_heads;
    int gw = 1;  // query heads per workgroup: the largest divisor of the group that fits 16 MFMA columns
    for (int c = 1; c <= 16 && c <= plan->group; ++c)
        if (plan->group % c == 0) gw = c;
    plan->heads_per_wg = gw;
    plan->hgroups = p->n_kv_heads * (plan->group / gw);
    int cap = p->max_context;
    const int64_t table_cap = (int64_t)p->max_pages_per_seq * p->page_size;
    if (table_cap < cap) cap = (int)table_cap;
    if (cap < 0) cap = 0;
    const int64_t tiles_max = ((int64_t)cap + kTok - 1) / kTok;
    plan->per = kDecodeMinTilesPerRange;
    // a unit of T tiles overlaps at most ceil(T / per) + 1 ranges, per >= the minimum
    plan->max_splits = (int)((tiles_max + plan->per - 1) / plan->per + 1);
    // page ids of a range's piece must fit the kernel's page-id buffer
    const int64_t fit = (int64_t)(kPgCap - 2) * p->page_size / kTok;
    plan->per_max = (int)(fit < kDecodeMaxTilesPerRange ? (fit > plan->per ? fit : plan->per) : kDecodeMaxTilesPerRange);
    plan->grid = decode_slots(p->head_dim, p->kv_dtype == ATTN_BF16);
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
    a.ctx_cap = cap < 0 ? 0 : cap;
    a.hgroups = plan->hgroups;
    a.per_min = plan->per;
    a.per_max = plan->per_max;
    a.slots = (int)plan->grid;
    a.max_splits = plan->max_splits;
    a.score_scale = p->scale * kLog2e;
    int shift = -1;
    for (int k = 0; k < 31; ++k)
        if ((1 << k) == p->page_size) shift = k;
    a.page_shift = shift;
    const bool bf16 = p->kv_dtype == ATTN_BF16;
    switch (p->head_dim) {
    case 128: return bf16 ? launch_typed<128, true>(a, plan->grid, stream) : launch_typed<128, false>(a, plan->grid, stream);
    case 256: return bf16 ? launch_typed<256, true>(a, plan->grid, stream) : launch_typed<256, false>(a, plan->grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
