// verify.hip -- pack-free DFlash2 block-verify attention on gfx950.
//
// Computes what the block-verify step computes with its pack kernel, its mask
// kernel and a masked GQA attention over the packed buffers (mlx-native
// 0.21.1, src/ops/dflash2_attention_pack.rs: the pack kernel's key order and
// bf16 rounding, the mask kernel's visibility rule), without materialising
// the packed Q/K/V or the mask.  For lane b with cache length L and write
// position wp:
//   keys     the `rows` drafted rows (bf16 of the current K/V), then ring slot
//            (wp - 1 - j) mod window for j = 0, 1, ... (newest first);
//   visible  query row i sees every drafted row and the cached rows
//            j < min(L, window - 1 - i);
//   scores   scale * (bf16(current Q) . K), softmax over the visible keys,
//   output   O f32 [lanes, q_heads, rows, head_dim].
//
// Design: the step is bound by HBM reads of the ring's visible rows (each is
// read once for all g * rows query rows of its KV head), so the kernel
// streams key tiles and keeps the arithmetic on the matrix cores.
//  * Workgroup (split, KV head x query-head group, lane) walks a contiguous
//    run of key tiles; up to 64 query columns (heads_per_wg heads x rows) sit
//    in 16-column slices, one per wave, all sharing the staged tiles.  The
//    splits per lane are sized on the device from the lanes' cache lengths so
//    the grid has about `target_wgs` busy workgroups whatever the lengths; a
//    second kernel merges the splits with a log-sum-exp reduction.
//  * Tile 0 of a lane is the drafted rows, converted to bf16 into LDS; ring
//    tiles are gathered row by row (the ring order wraps) with
//    global_load_lds_dwordx4 into a ring of XOR-swizzled LDS stages, several
//    tiles ahead of the one in use.
//  * The per-tile step (attend.h): S^T = K Q^T and O^T += V^T P^T as
//    v_mfma_f32_16x16x32, P as a bf16 hi + lo pair.  Only tiles that reach
//    past the shortest row's frontier evaluate the mask.
#include <math.h>

#include "attend.h"
#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void;

struct VerifyArgs {
    const uint16_t *ring_k, *ring_v;
    const float *cur_q, *cur_k, *cur_v;
    const uint32_t *cache_lengths, *write_positions;
    float *o;
    float *part;    // [lanes][q_heads][rows][max_splits][D]
    float2 *ml;     // [lanes][q_heads][rows][max_splits]
    int lanes, q_heads, kv_heads, rows, window;
    int group, heads_per_wg, qgroups, ncols;
    int max_splits, target_wgs;
    float score_scale;  // scale * log2(e)
};

// Ring rows any query row of lane b sees: min(L, window - 1).
__device__ __forceinline__ int reach_of(const VerifyArgs &a, int b) {
    const uint32_t len = a.cache_lengths[b];
    const uint32_t cap = (uint32_t)a.window - 1u;
    return (int)(len < cap ? len : cap);
}

// Work split: per lane, its tiles (drafted tile + ring tiles), tiles per split
// and splits; `items` = every (lane, KV head x query-head group, split) in
// lane-major order.  Every workgroup and the merge kernel derive the same
// numbers from the cache lengths.
struct Split {
    int tiles[4], tps[4], splits[4];
    int items;
};
// x[i] for a small register array and a wave-uniform i < 4, without dynamic indexing
__device__ __forceinline__ int pick4(const int (&x)[4], int i) {
    return i == 0 ? x[0] : (i == 1 ? x[1] : (i == 2 ? x[2] : x[3]));
}
template <int TK>
__device__ __forceinline__ Split split_all(const VerifyArgs &a) {
    Split sp;
    int total = 0, most = 1;
    for (int x = 0; x < 4; ++x) {
        sp.tiles[x] = x < a.lanes ? 1 + (reach_of(a, x) + TK - 1) / TK : 0;
        total += sp.tiles[x];
        most = sp.tiles[x] > most ? sp.tiles[x] : most;
    }
    const int units = a.kv_heads * a.qgroups;
    // the fewest tiles per split that keeps the work items within target_wgs (one
    // round on the chip), with at most max_splits splits per lane
    int tps = (total * units + a.target_wgs - 1) / a.target_wgs;
    tps = tps > 1 ? tps : 1;
    for (;; ++tps) {
        int items = 0;
        for (int x = 0; x < 4; ++x) {
            const int cap = (sp.tiles[x] + a.max_splits - 1) / a.max_splits;
            sp.tps[x] = tps > cap ? tps : cap;
            sp.splits[x] = (sp.tiles[x] + sp.tps[x] - 1) / sp.tps[x];
            items += sp.splits[x];
        }
        sp.items = items * units;
        if (sp.items <= a.target_wgs || tps >= most) break;
    }
    return sp;
}

// Gather ring tile t (ring rows j = TK*(t-1) .. TK*t - 1, clamped to the last
// visible row) of one KV head into an LDS stage.  Each global_load_lds_dwordx4
// fills 64 consecutive 16-byte slots from M0; the waves split the slots.
template <int D, int TK, int NWV>
__device__ __forceinline__ void issue_ring(const uint16_t *ring_k, const uint16_t *ring_v, uint16_t *k_tile,
                                           uint16_t *v_tile, int t, int reach0, int wp, int window, int wave,
                                           int lane) {
    constexpr int CH = D / 8;
    constexpr int NLD = TK * CH / (64 * NWV);
    const uint32_t kb = (uint32_t)(uintptr_t)(lds_void *)k_tile;
    const uint32_t vb = (uint32_t)(uintptr_t)(lds_void *)v_tile;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int slot = (i * NWV + wave) * 64 + lane;
        const int row = slot / CH, pch = slot % CH;
        int j = TK * (t - 1) + row;
        j = j < reach0 ? j : reach0 - 1;
        int rs = wp + window - 1 - j;  // in [wp, wp + window - 1]
        rs = rs >= window ? rs - window : rs;
        const int64_t off = (int64_t)rs * D;
        const uint16_t *ksrc = ring_k + off + 8 * (pch ^ attend_k_swz(row));
        const uint16_t *vsrc = ring_v + off + 8 * (pch ^ attend_v_swz(row));
        const uint32_t mk = __builtin_amdgcn_readfirstlane(kb + (i * NWV + wave) * 1024);
        const uint32_t mv = __builtin_amdgcn_readfirstlane(vb + (i * NWV + wave) * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(mk), "v"(ksrc) : "memory");
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(mv), "v"(vsrc) : "memory");
    }
}

__device__ __forceinline__ uint4v f32x8_to_bf16(const float *src) {
    const float4v x0 = *reinterpret_cast<const float4v *>(src);
    const float4v x1 = *reinterpret_cast<const float4v *>(src + 4);
    return uint4v{pack2(f32_to_bf16_rne(x0[0]), f32_to_bf16_rne(x0[1])),
                  pack2(f32_to_bf16_rne(x0[2]), f32_to_bf16_rne(x0[3])),
                  pack2(f32_to_bf16_rne(x1[0]), f32_to_bf16_rne(x1[1])),
                  pack2(f32_to_bf16_rne(x1[2]), f32_to_bf16_rne(x1[3]))};
}

// Tile 0: drafted rows p < rows as bf16, rows past them zero (masked anyway).
template <int D, int TK, int NWV>
__device__ __forceinline__ void write_drafted(const VerifyArgs &a, int b, int kh, uint16_t *k_tile,
                                              uint16_t *v_tile) {
    constexpr int CH = D / 8;
    for (int slot = threadIdx.x; slot < TK * CH; slot += 64 * NWV) {
        const int row = slot / CH, pch = slot % CH;
        uint4v kv = uint4v{0u, 0u, 0u, 0u}, vv = kv;
        if (row < a.rows) {
            const int64_t src = (((int64_t)b * a.rows + row) * a.kv_heads + kh) * D;
            kv = f32x8_to_bf16(a.cur_k + src + 8 * (pch ^ attend_k_swz(row)));
            vv = f32x8_to_bf16(a.cur_v + src + 8 * (pch ^ attend_v_swz(row)));
        }
        *reinterpret_cast<uint4v *>(k_tile + row * D + 8 * pch) = kv;
        *reinterpret_cast<uint4v *>(v_tile + row * D + 8 * pch) = vv;
    }
}

// Keys per tile and the LDS ring.  At head_dim 128 two teams of waves take
// alternate tiles (two waves per SIMD hide each other's latencies); the ring
// holds NGRP groups of TEAMS tiles: one group in use, NGRP - 1 in flight.
template <int D>
struct VerifyTiling {
    static constexpr int TK = kVerifyTileKeys;
    static constexpr int TEAMS = D == 128 ? 2 : 1;
    static constexpr int NGRP = D == 128 ? 3 : 2;
};

template <int D, int NWV>
__global__ __launch_bounds__(64 * NWV * VerifyTiling<D>::TEAMS) void verify_partial_kernel(VerifyArgs a) {
    constexpr int TK = VerifyTiling<D>::TK;          // keys per tile
    constexpr int TEAMS = VerifyTiling<D>::TEAMS;    // tiles processed side by side
    constexpr int NGRP = VerifyTiling<D>::NGRP;      // groups of TEAMS tiles in the LDS ring
    constexpr int NSTAGE = TEAMS * NGRP;
    constexpr int NW = TEAMS * NWV;                  // waves: TEAMS teams of NWV 16-column slices
    constexpr int TILE = TK * D;                     // elements of one K (or V) tile
    constexpr int KSTEPS = D / 32;                   // MFMA k-steps of S^T
    constexpr int DBLK = D / 16;                     // 16-row blocks of O^T
    constexpr int NLD = TK * (D / 8) / (64 * NW);    // loads per wave per K (or V) tile
    static_assert((TK * (D / 8)) % (64 * NW) == 0, "tile slots must split evenly over the waves");
    static_assert(TEAMS * (NGRP - 1) <= 6 && TEAMS * (NGRP - 1) * 2 * NLD <= 63, "vmcnt immediates");
    static_assert(TEAMS == 1 || NWV * (DBLK * 64 * 16 + 64 * 8) <= NSTAGE * 2 * TILE * 2, "team exchange fits the ring");
    __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[NSTAGE * 2 * TILE];  // [stage][K, V]

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int team = wave / NWV, cw = wave % NWV;
    const Split sp = split_all<TK>(a);
    const int units = a.kv_heads * a.qgroups;
    // work items are numbered densely so consecutive workgroups (which the
    // dispatcher deals round-robin to the XCDs) all have work
    for (int item = blockIdx.x; item < sp.items; item += gridDim.x) {
        int b = 0, rest = item;
#pragma unroll
        for (int x = 0; x < 3; ++x)
            if (b == x && rest >= sp.splits[x] * units) {
                rest -= sp.splits[x] * units;
                b = x + 1;
            }
        const int nspl = pick4(sp.splits, b), tps = pick4(sp.tps, b);
        const int unit = rest / nspl, split = rest % nspl;
        const int kh = unit / a.qgroups, qg = unit % a.qgroups;
        const int t_begin = split * tps;
        const int t_end = min(t_begin + tps, pick4(sp.tiles, b));
        const int reach0 = reach_of(a, b);
        const uint32_t len = a.cache_lengths[b];
        const int wp = (int)(a.write_positions[b] % (uint32_t)a.window);
        // shortest frontier over the rows: tiles ending at or before it need no mask
        const int reach_min = (int)min(len, (uint32_t)(a.window - a.rows));

        const int64_t head_off = ((int64_t)b * a.kv_heads + kh) * a.window * D;
        const uint16_t *ring_k = a.ring_k + head_off;
        const uint16_t *ring_v = a.ring_v + head_off;

        // query column of this lane: (head of the group, row)
        const int slot = lane & 15, g4 = lane >> 4;
        const int col = 16 * cw + slot;
        const bool col_ok = col < a.ncols;
        const int hh = col_ok ? col / a.rows : 0, qi = col_ok ? col % a.rows : 0;
        const int head = kh * a.group + qg * a.heads_per_wg + hh;
        const int reach_col = (int)min(len, (uint32_t)(a.window - 1 - qi));

        // Q rows first (idle columns read column 0's row), then the first ring tiles; Q is
        // waited for explicitly, so it does not queue behind the tiles.  The loads are
        // issued from inline asm (their registers are written when vmcnt says so), and the
        // empty asm after the wait ties every use of them to that wait.
        float4v x[2 * KSTEPS];
        {
            const float *qp = a.cur_q + (((int64_t)b * a.rows + qi) * a.q_heads + head) * D + 8 * g4;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x[2 * ks]) : "v"(qp + 32 * ks) : "memory");
                asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(x[2 * ks + 1]) : "v"(qp + 32 * ks + 4) : "memory");
            }
        }
        int n_pro = 0;  // ring tiles issued by the prologue: groups 0 .. NGRP - 2
#pragma unroll
        for (int k = 0; k < TEAMS * (NGRP - 1); ++k) {
            const int t = t_begin + k;
            if (t >= 1 && t < t_end) {
                uint16_t *st = kv_lds + k * 2 * TILE;
                issue_ring<D, TK, NW>(ring_k, ring_v, st, st + TILE, t, reach0, wp, a.window, wave, lane);
                ++n_pro;
            }
        }
        attend_wait_tiles<2 * NLD>(n_pro);
#pragma unroll
        for (int i = 0; i < 2 * KSTEPS; ++i) asm volatile("" : "+v"(x[i]));

        // Q^T as the B operand of S^T = K Q^T: column = lane % 16, k = 32*ks + 8*(lane/16) + e
        uint4v qf[KSTEPS];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const float4v x0 = x[2 * ks], x1 = x[2 * ks + 1];
            qf[ks] = uint4v{pack2(f32_to_bf16_rne(x0[0]), f32_to_bf16_rne(x0[1])),
                            pack2(f32_to_bf16_rne(x0[2]), f32_to_bf16_rne(x0[3])),
                            pack2(f32_to_bf16_rne(x1[0]), f32_to_bf16_rne(x1[1])),
                            pack2(f32_to_bf16_rne(x1[2]), f32_to_bf16_rne(x1[3]))};
            if (!col_ok) qf[ks] = uint4v{0u, 0u, 0u, 0u};
        }
        if (t_begin == 0) write_drafted<D, TK, NW>(a, b, kh, kv_lds, kv_lds + TILE);

        float4v acc[DBLK];
#pragma unroll
        for (int db = 0; db < DBLK; ++db) acc[db] = float4v{0.f, 0.f, 0.f, 0.f};
        float m_run = -INFINITY, l_run = 0.f;

        const int ngroups = (t_end - t_begin + TEAMS - 1) / TEAMS;
        int gstage = 0;  // first stage of the group in use
        for (int k = 0; k < ngroups; ++k) {
            // ring tiles issued after group k: up to the end of group k + NGRP - 2
            const int issued_end = min(t_end, t_begin + TEAMS * (k + NGRP - 1));
            const int after = max(0, issued_end - (t_begin + TEAMS * (k + 1)));
            attend_wait_tiles<2 * NLD>(after);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave's part of group k is in
            {
                // group k + NGRP - 1 goes into the stages of group k - 1: every wave is past it
                const int sn = gstage == 0 ? NSTAGE - TEAMS : gstage - TEAMS;
#pragma unroll
                for (int e = 0; e < TEAMS; ++e) {
                    const int tn = t_begin + TEAMS * (k + NGRP - 1) + e;
                    if (tn < t_end) {
                        uint16_t *st = kv_lds + (sn + e) * 2 * TILE;
                        issue_ring<D, TK, NW>(ring_k, ring_v, st, st + TILE, tn, reach0, wp, a.window, wave, lane);
                    }
                }
            }
            const int t = t_begin + TEAMS * k + team;
            if (t < t_end) {
                // tile 0 is the drafted rows (keys p < rows visible to every column); ring
                // tile t holds keys j = TK*(t-1) + k, visible to a column while j < its reach
                const uint16_t *k_tile = kv_lds + (gstage + team) * 2 * TILE;
                attend_tile<D, TK, true, false>(k_tile, k_tile + TILE, qf, qf, a.score_scale,
                                                t == 0 || TK * t > reach_min, t == 0 ? 0 : TK * (t - 1),
                                                t == 0 ? a.rows : reach_col, acc, m_run, l_run, lane);
            }
            gstage = gstage + TEAMS == NSTAGE ? 0 : gstage + TEAMS;
        }

        // ---- merge the teams' states through LDS (the ring is free once every wave is here)
        if constexpr (TEAMS == 2) attend_merge_teams<D, NWV>(kv_lds, team, cw, lane, acc, m_run, l_run);

        // ---- this split's unnormalised O and (m, l) per column
        if (team == 0 && col_ok) {
            const int64_t u = (((int64_t)b * a.q_heads + head) * a.rows + qi) * a.max_splits + split;
            float *dst = a.part + u * D + 4 * g4;
#pragma unroll
            for (int db = 0; db < DBLK; ++db) *reinterpret_cast<float4v *>(dst + 16 * db) = acc[db];
            if (g4 == 0) a.ml[u] = make_float2(m_run, l_run);
        }
        __syncthreads();  // the next item's prologue refills the stages
    }
}

// One wave per (lane, query head, row): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// The (m, l) of every split slot (lane s holding slot s) and the first NP O slices are
// requested together with the cache lengths that give the split count, so a row of at
// most NP splits costs one memory round trip; slots past the count are never used.
template <int D>
__global__ __launch_bounds__(256) void verify_merge_kernel(VerifyArgs a) {
    constexpr int TK = VerifyTiling<D>::TK;
    constexpr int PER_LANE = D / 64;
    constexpr int NP = 8;  // splits whose slices are loaded up front
    static_assert(kVerifyMaxSplits <= 64, "one split per lane");
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (unit >= (int64_t)a.lanes * a.q_heads * a.rows) return;
    const int b = (int)(unit / ((int64_t)a.q_heads * a.rows));
    const float2 *ml = a.ml + unit * a.max_splits;
    const float *part = a.part + unit * a.max_splits * D + lane * PER_LANE;
    const float2 my0 = lane < a.max_splits ? ml[lane] : make_float2(-INFINITY, 0.f);
    float v[NP][PER_LANE];
#pragma unroll
    for (int j = 0; j < NP; ++j)
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) v[j][i] = j < a.max_splits ? part[(int64_t)j * D + i] : 0.f;
    const int nsplit = pick4(split_all<TK>(a).splits, b);

    // every split below nsplit wrote its partial (zeros where it saw no key)
    const float2 my = lane < nsplit ? my0 : make_float2(-INFINITY, 0.f);
    float mmax = my.x;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off));
    const float w = my.x == -INFINITY ? 0.f : exp2f(my.x - mmax);  // splits with no visible key weigh 0
    float lsum = w * my.y;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lsum += __shfl_xor(lsum, off);
    float o[PER_LANE];
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) o[i] = 0.f;
#pragma unroll
    for (int j = 0; j < NP; ++j) {
        const float wj = __shfl(w, j);
        if (j < nsplit) {
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) o[i] = fmaf(wj, v[j][i], o[i]);
        }
    }
    for (int j = NP; j < nsplit; ++j) {
        const float wj = __shfl(w, j);
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) o[i] = fmaf(wj, part[(int64_t)j * D + i], o[i]);
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float *orow = a.o + unit * D + lane * PER_LANE;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) orow[i] = o[i] * inv;
}

template <int D, int NWV>
hipError_t launch_typed(const VerifyArgs &a, hipStream_t stream) {
    dim3 grid(a.target_wgs);
    hipLaunchKernelGGL((verify_partial_kernel<D, NWV>), grid, dim3(64 * NWV * VerifyTiling<D>::TEAMS), 0, stream,
                       a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t units = (int64_t)a.lanes * a.q_heads * a.rows;
    hipLaunchKernelGGL((verify_merge_kernel<D>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const VerifyArgs &a, hipStream_t stream) {
    const int waves = (a.ncols + 15) / 16;
    if (waves <= 1) return launch_typed<D, 1>(a, stream);
    if (waves <= 2) return launch_typed<D, 2>(a, stream);
    return launch_typed<D, 4>(a, stream);
}

}  // namespace

// One workgroup per CU of the current device: the LDS ring takes most of a CU's LDS.
int verify_target_workgroups() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        return kVerifyDefaultWorkgroups;
    return cus;
}

int plan_verify(const dflash_params *p, VerifyPlan *plan) {
    const int group = (int)(p->q_heads / p->kv_heads);
    int gw = 1;  // query heads per workgroup: the largest divisor of the group whose rows fit 64 columns
    for (int c = 1; c <= group && c * (int)p->rows <= 64; ++c)
        if (group % c == 0) gw = c;
    plan->group = group;
    plan->heads_per_wg = gw;
    plan->qgroups = group / gw;
    const int tk = kVerifyTileKeys;
    const int64_t tiles = 1 + ((int64_t)p->window - 1 + tk - 1) / tk;
    plan->max_splits = (int)(tiles < kVerifyMaxSplits ? tiles : kVerifyMaxSplits);
    plan->target_wgs = verify_target_workgroups();
    const size_t units = (size_t)p->lanes * p->q_heads * p->rows;
    plan->ml_offset = 0;
    plan->ml_bytes = units * plan->max_splits * sizeof(float2);
    plan->part_offset = (plan->ml_bytes + 255) & ~(size_t)255;
    plan->part_bytes = units * plan->max_splits * p->head_dim * sizeof(float);
    plan->workspace_bytes = plan->part_offset + plan->part_bytes;
    return ATTN_OK;
}

hipError_t launch_dflash_verify(const dflash_params *p, const VerifyPlan *plan, float scale, const uint16_t *ring_k,
                                const uint16_t *ring_v, const float *cur_q, const float *cur_k, const float *cur_v,
                                const uint32_t *cache_lengths, const uint32_t *write_positions, float *o, void *ws,
                                hipStream_t stream) {
    VerifyArgs a;
    a.ring_k = ring_k;
    a.ring_v = ring_v;
    a.cur_q = cur_q;
    a.cur_k = cur_k;
    a.cur_v = cur_v;
    a.cache_lengths = cache_lengths;
    a.write_positions = write_positions;
    a.o = o;
    a.ml = (float2 *)((uint8_t *)ws + plan->ml_offset);
    a.part = (float *)((uint8_t *)ws + plan->part_offset);
    a.lanes = (int)p->lanes;
    a.q_heads = (int)p->q_heads;
    a.kv_heads = (int)p->kv_heads;
    a.rows = (int)p->rows;
    a.window = (int)p->window;
    a.group = plan->group;
    a.heads_per_wg = plan->heads_per_wg;
    a.qgroups = plan->qgroups;
    a.ncols = plan->heads_per_wg * (int)p->rows;
    a.max_splits = plan->max_splits;
    a.target_wgs = plan->target_wgs;
    a.score_scale = scale * kLog2e;
    switch (p->head_dim) {
    case 128: return launch_dim<128>(a, stream);
    case 256: return launch_dim<256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
