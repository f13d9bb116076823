// attend.h -- the per-tile step shared by the multi-column split-KV attention
// kernels (pack-free block verify, multi-token paged attention): up to 16
// query columns per wave against a tile of keys staged in LDS.
//
//  * S^T = K Q^T and O^T += V^T P^T run as v_mfma_f32_16x16x32: lane l holds
//    column l % 16 and keys 16*blk + 4*(l/16) + r of the tile; P^T goes from
//    the S^T accumulators into the B operand, V^T fragments come from
//    ds_read_b64_tr_b16 on row-major V.
//  * Online softmax in log2 units with a lazy reference max: the max moves
//    only when a tile's max passes it by more than 2^8, so the accumulators
//    are rarely rescaled (P then stays below 256).
//  * P enters the PV product as a hi + lo pair of the K/V type (two
//    products), about 16 significant bits, so rows that see few keys keep
//    the accuracy of the f32 softmax.
#pragma once

#include <math.h>

#include "device_common.h"

namespace attn {

constexpr float kAttendLazyRescale = 8.f;  // log2 units

typedef __attribute__((address_space(3))) short4v attend_lds_short4;

template <bool BF16>
__device__ __forceinline__ float4v attend_mfma(uint4v a, uint4v b, float4v c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bhalf8, a), __builtin_bit_cast(bhalf8, b),
                                                       c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a), __builtin_bit_cast(half8, b), c,
                                                      0, 0, 0);
    }
}

// (x[l], x[l ^ 16]) then (x[l], x[l ^ 32]): the four lanes holding one column
__device__ __forceinline__ float attend_col_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    return max_with_other_half(x);
}
__device__ __forceinline__ float attend_col_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    return sum_with_other_half(x);
}

// LDS tile layouts (TK key rows x D, chunks of 16 bytes):
//  K: logical chunk c of row r at physical c ^ (r % 16)   (A-operand reads: 16 rows, one chunk)
//  V: logical chunk c of row r at physical c ^ 2*(r % 8)   (transposing reads: 8 rows x 2 chunks)
__device__ __forceinline__ int attend_k_swz(int row) { return row & 15; }
__device__ __forceinline__ int attend_v_swz(int row) { return (row & 7) << 1; }

// p as a hi part and the remainder, both of the K/V type, packed two per dword
// by the caller: bf16 keeps the upper half of the f32 bits, f16 rounds.
template <bool BF16>
__device__ __forceinline__ void attend_split_p(float p, uint32_t &hi, uint32_t &lo) {
    if constexpr (BF16) {
        hi = __float_as_uint(p) & 0xffff0000u;
        lo = __float_as_uint(p - __uint_as_float(hi)) & 0xffff0000u;
        hi >>= 16;
        lo >>= 16;
    } else {
        const _Float16 h = (_Float16)p;
        const _Float16 l = (_Float16)(p - (float)h);
        hi = __builtin_bit_cast(uint16_t, h);
        lo = __builtin_bit_cast(uint16_t, l);
    }
}

// One tile of TK keys for this wave's 16 columns.
//  qf, qlo    B fragments of Q^T (qlo used when QLO: a second product carrying the
//             rest of an f32 Q the K/V type cannot hold)
//  s_mul      factor applied to S (1 when Q is prescaled)
//  key0       key index of tile row 0; masked: key k of the tile is visible to this
//             lane's column iff key0 + k < limit
//  acc, m_run, l_run   this lane's column state (m in log2 units)
template <int D, int TK, bool BF16, bool QLO>
__device__ __forceinline__ void attend_tile(const uint16_t *k_tile, const uint16_t *v_tile, const uint4v (&qf)[D / 32],
                                            const uint4v (&qlo)[D / 32], float s_mul, bool masked, int key0,
                                            int limit, float4v (&acc)[D / 16], float &m_run, float &l_run, int lane) {
    constexpr int KSTEPS = D / 32;  // MFMA k-steps of S^T
    constexpr int DBLK = D / 16;    // 16-row blocks of O^T
    constexpr int KBLK = TK / 16;   // 16-key blocks of S^T
    constexpr int PSTEPS = TK / 32; // 32-key k-steps of O^T
    const int slot = lane & 15, g4 = lane >> 4;

    // ---- S^T: every K fragment of the tile is read before the first product, and
    // the V^T fragments before the softmax, so the LDS latency overlaps other work
    uint4v kf[KBLK][KSTEPS];
#pragma unroll
    for (int blk = 0; blk < KBLK; ++blk) {
        const int row = 16 * blk + slot;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
            kf[blk][ks] =
                *reinterpret_cast<const uint4v *>(k_tile + row * D + 8 * ((4 * ks + g4) ^ attend_k_swz(row)));
    }
    float4v s[KBLK];
#pragma unroll
    for (int blk = 0; blk < KBLK; ++blk) s[blk] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int blk = 0; blk < KBLK; ++blk) {
            s[blk] = attend_mfma<BF16>(kf[blk][ks], qf[ks], s[blk]);
            if constexpr (QLO) s[blk] = attend_mfma<BF16>(kf[blk][ks], qlo[ks], s[blk]);
        }
    lds_ahead_schedule<KBLK * KSTEPS, 1, QLO ? 2 : 1, KBLK * KSTEPS>();
    // V^T fragments (A operand), 32 keys per k-step: k slot e < 4 <-> key 32*ps + 4*g4 + e,
    // e >= 4 <-> key 32*ps + 16 + 4*g4 + (e - 4).  A 16-lane group reads rows kb..kb+3 x
    // 16 columns per ds_read_b64_tr_b16: lane j points at row kb + j/4, columns
    // 16*db + 4*(j%4), and receives rows kb..kb+3 of column 16*db + j.
    const int v_rsub = lane & 15;
    uint4v vf[PSTEPS][DBLK];
#pragma unroll
    for (int pstep = 0; pstep < PSTEPS; ++pstep) {
        const int r0 = 32 * pstep + 4 * g4 + (v_rsub >> 2), r1 = r0 + 16;
        const uint16_t *v0 = v_tile + r0 * D + 4 * (v_rsub & 1);
        const uint16_t *v1 = v_tile + r1 * D + 4 * (v_rsub & 1);
        const int c0 = (v_rsub & 3) >> 1;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            const int lch = 2 * db + c0;
            const short4v lo =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((attend_lds_short4 *)(v0 + 8 * (lch ^ attend_v_swz(r0))));
            const short4v hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((attend_lds_short4 *)(v1 + 8 * (lch ^ attend_v_swz(r1))));
            vf[pstep][db] = uint4v{pack2((uint16_t)lo[0], (uint16_t)lo[1]), pack2((uint16_t)lo[2], (uint16_t)lo[3]),
                                   pack2((uint16_t)hi[0], (uint16_t)hi[1]), pack2((uint16_t)hi[2], (uint16_t)hi[3])};
        }
    }
    if (s_mul != 1.f) {
#pragma unroll
        for (int blk = 0; blk < KBLK; ++blk) s[blk] *= s_mul;
    }
    if (masked) {
        const int k0 = key0 + 4 * g4;
#pragma unroll
        for (int blk = 0; blk < KBLK; ++blk)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (k0 + 16 * blk + r >= limit) s[blk][r] = -INFINITY;
    }

    // ---- online softmax per column (16 keys here, the rest in lanes ^16, ^32, ^48)
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < KBLK; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[blk][r]);
    mx = attend_col_max(mx);
    const bool grow = mx > m_run + kAttendLazyRescale;
    if (__ballot(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;  // 0 when m_run = -inf
        m_run = grow ? mx : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) acc[db] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // a column that has seen no visible key yet
    uint32_t phi[4 * KBLK], plo[4 * KBLK];
    float ps = 0.f;
#pragma unroll
    for (int blk = 0; blk < KBLK; ++blk)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(s[blk][r] - m_use);
            ps += p;
            attend_split_p<BF16>(p, phi[4 * blk + r], plo[4 * blk + r]);
        }
    l_run += attend_col_sum(ps);

    // ---- O^T[d][col] += V^T[d][key] P^T[key][col]
#pragma unroll
    for (int pstep = 0; pstep < PSTEPS; ++pstep) {
        uint4v pb, pl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pb[e] = phi[8 * pstep + 2 * e] | (phi[8 * pstep + 2 * e + 1] << 16);
            pl[e] = plo[8 * pstep + 2 * e] | (plo[8 * pstep + 2 * e + 1] << 16);
        }
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
            acc[db] = attend_mfma<BF16>(vf[pstep][db], pb, acc[db]);
            acc[db] = attend_mfma<BF16>(vf[pstep][db], pl, acc[db]);
        }
    }
}

// Merge the column state of team 1 into team 0 through LDS (xch: NWV * (DBLK*64*16 +
// 64*8) bytes, free of other use).  Every wave of the workgroup calls it.
template <int D, int NWV>
__device__ __forceinline__ void attend_merge_teams(void *xch, int team, int cw, int lane, float4v (&acc)[D / 16],
                                                   float &m_run, float &l_run) {
    constexpr int DBLK = D / 16;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float4v *x_acc = reinterpret_cast<float4v *>(xch);  // [slice][db][lane]
    float2 *x_ml = reinterpret_cast<float2 *>(x_acc + NWV * DBLK * 64);
    if (team == 1) {
#pragma unroll
        for (int db = 0; db < DBLK; ++db) x_acc[(cw * DBLK + db) * 64 + lane] = acc[db];
        x_ml[cw * 64 + lane] = make_float2(m_run, l_run);
    }
    __syncthreads();
    if (team == 0) {
        const float2 o = x_ml[cw * 64 + lane];
        const float m = fmaxf(m_run, o.x);
        const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
        const float a1 = o.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(o.x - m);
#pragma unroll
        for (int db = 0; db < DBLK; ++db) acc[db] = acc[db] * a0 + x_acc[(cw * DBLK + db) * 64 + lane] * a1;
        l_run = l_run * a0 + o.y * a1;
        m_run = m;
    }
}

// s_waitcnt vmcnt(n * PER) for n <= 6, the count a compile-time immediate
template <int PER>
__device__ __forceinline__ void attend_wait_tiles(int n) {
    switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * PER) : "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(5 * PER) : "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * PER) : "memory"); break;
    }
}

}  // namespace attn
