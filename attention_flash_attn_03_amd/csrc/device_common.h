// device_common.h -- small device helpers shared by the gfx950 kernels:
// vector types, 16-bit float conversions and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace attn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bhalf8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));

// f32 -> bf16 bits, round to nearest with ties to even; NaN stays NaN with
// its quiet bit set; overflow rounds to infinity; subnormals are kept.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// Pack two 16-bit patterns into one dword (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) {
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Exchange with the lane 32 positions away: returns {x[l], x[l^32]} in an
// order that depends on the half; max/sum of the pair is symmetric.
__device__ __forceinline__ float max_with_other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_other_half(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 16 lanes of a row (lanes 16k..16k+15); every lane gets the sum.
// DPP: swap neighbours, swap pairs, mirror within 8, mirror within 16.
__device__ __forceinline__ float row16_sum(float x) {
    x += __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
    x += __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
    x += __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x141, 0xF, 0xF, true)); // row_half_mirror
    x += __uint_as_float(__builtin_amdgcn_mov_dpp(__float_as_uint(x), 0x140, 0xF, 0xF, true)); // row_mirror
    return x;
}

// Scheduling pattern for a run of N MFMAs that each consume R LDS reads issued in
// the same block: the reads of the first A MFMAs go first, then every MFMA (M of
// them per operand group) is followed by the reads of the group A ahead, so the
// LDS latency hides under the matrix cores instead of stalling each MFMA.
template <int N, int R, int M, int A>
__device__ __forceinline__ void lds_ahead_schedule() {
    __builtin_amdgcn_sched_group_barrier(0x100, R * A, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < N - A; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, M, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M * A, 0);
}

// N steps, each an MFMA group whose operand T is read from LDS: the read of step
// i + DIST is issued before the MFMAs of step i, with scheduling fences that keep
// this order, so every operand has its own registers and the wait before step i
// covers only its own read while DIST more are in flight.
template <int N, int DIST, typename T, typename Load, typename Use>
__device__ __forceinline__ void lds_pipeline(Load &&load, Use &&use) {
    T f[DIST + 1];
#pragma unroll
    for (int i = 0; i < DIST && i < N; ++i) f[i] = load(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if (i + DIST < N) f[(i + DIST) % (DIST + 1)] = load(i + DIST);
        __builtin_amdgcn_sched_barrier(0);
        use(i, f[i % (DIST + 1)]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Log-sum-exp merge of nsplit partials of one output row, one wave:
//   o = sum_s 2^(m_s - M) O_s,  lsum = sum_s 2^(m_s - M) l_s,  M = max_s m_s
// ml[s] = (m_s, l_s) (m in log2 units, -inf for a piece that saw no key, whose
// O_s is 0); O_s is part[s*D + d], lane l holding d = l*PER + i.  The (m, l) of
// the first 64 pieces and the first eight O slices are loaded together, so a row
// of at most eight pieces costs one memory round trip.
template <int D>
__device__ __forceinline__ void merge_pieces(const float2 *ml, const float *part, int nsplit, int lane,
                                             float (&o)[D / 64], float &lsum) {
    constexpr int PER = D / 64;
    part += lane * PER;
    const float2 my0 = lane < nsplit ? ml[lane] : make_float2(-INFINITY, 0.f);
    float v0[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < PER; ++i) v0[u][i] = u < nsplit ? part[(int64_t)u * D + i] : 0.f;
    float mmax = my0.x;
    for (int s = 64 + lane; s < nsplit; s += 64) mmax = fmaxf(mmax, ml[s].x);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off));
#pragma unroll
    for (int i = 0; i < PER; ++i) o[i] = 0.f;
    lsum = 0.f;
    if (mmax == -INFINITY) return;  // no piece saw a key
    for (int s0 = 0; s0 < nsplit; s0 += 64) {
        const float2 my = s0 == 0 ? my0 : (s0 + lane < nsplit ? ml[s0 + lane] : make_float2(-INFINITY, 0.f));
        const float w = my.x == -INFINITY ? 0.f : exp2f(my.x - mmax);
        float lw = w * my.y;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) lw += __shfl_xor(lw, off);
        lsum += lw;
        const int n = min(64, nsplit - s0);
        for (int j = 0; j < n; j += 8) {
            float v[8][PER];
            if (s0 == 0 && j == 0) {
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int i = 0; i < PER; ++i) v[u][i] = v0[u][i];
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int i = 0; i < PER; ++i) v[u][i] = j + u < n ? part[(int64_t)(s0 + j + u) * D + i] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float wj = __shfl(w, (j + u) & 63);  // zero past n: those slices were loaded as 0
#pragma unroll
                for (int i = 0; i < PER; ++i) o[i] = fmaf(wj, v[u][i], o[i]);
            }
        }
    }
}

}  // namespace attn
