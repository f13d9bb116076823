// paged_prefill.hip -- multi-token attention over a paged KV cache on gfx950.
//
// What is computed follows ferrum-kernels 0.8.3,
// src/backend/metal/vnext_ops/causal_attention.rs (the attention dispatch
// over fixed-size KV pages read through a per-sequence page table, for
// `tokens` new tokens starting at `position_start`, causal; query head h reads
// KV head h / (query_heads / key_value_heads); the step writes the new
// tokens' K/V into the pages before attending):
//   query token i of sequence b sits at position start_b + i and attends to
//   the keys t <= start_b + i of its sequence.
// With one token at start = context - 1 it is the paged decode step; with
// many it is chunked prefill, or block verify straight from the page table.
//
// Design: the paged decode kernel's balanced line of 32-token tiles (every
// (sequence, KV head group) unit laid end to end, every workgroup the same
// number of tiles, pieces cut at unit boundaries, a log-sum-exp merge; the
// tiles per workgroup spread the line over one workgroup per CU), with
// the query tokens of a sequence as MFMA columns: up to 64 columns (heads x
// tokens of one KV head) per workgroup, 16 per wave, sharing K/V tiles staged
// in LDS.  The per-tile step is attend.h's; the causal frontier is evaluated
// only on tiles that reach past the first token's.
#include <math.h>

#include "attend.h"
#include "device_common.h"
#include "internal.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTK = 32;  // keys per tile
// What starting a piece costs (page ids, the first tiles' round trip, the epilogue), in
// tiles of the main loop: every unit occupies this many extra places on the line, so a
// workgroup whose range holds a unit's start gets that many fewer tiles.
constexpr int kPieceCostTiles = 8;
constexpr int kPgCap = kMultiMaxTilesPerWorkgroup * kTK + 2;  // page ids of one piece, any page size

typedef __attribute__((address_space(3))) void lds_void;

struct MultiArgs {
    const float *q;
    const uint16_t *k_pool, *v_pool;
    const int32_t *page_table, *query_lens, *position_starts;
    float *o;
    float *part;     // [batch][max_tokens][n_heads][max_splits][D]
    float2 *ml;      // [batch][max_tokens][n_heads][max_splits]
    int32_t *npiece; // [batch][hgroups]: pieces of the unit (written by its first piece)
    int64_t q_bs, q_ts, q_hs, o_bs, o_ts, o_hs, page_stride, token_stride, head_stride;
    int batch, n_heads, group, heads_per_wg, qgroups, hgroups, max_tokens, ncols;
    int page_size, page_shift, max_pages, num_pages, ctx_cap;
    int target;      // workgroups the line is spread over (one per CU)
    int max_splits;
    float score_scale;  // scale * log2(e)
};

struct SeqInfo {
    int tokens, start, ctx, tiles;
};

__device__ __forceinline__ SeqInfo seq_info(const MultiArgs &a, int b) {
    SeqInfo s;
    int t = a.query_lens[b];
    s.tokens = t < 0 ? 0 : (t > a.max_tokens ? a.max_tokens : t);
    int st = a.position_starts[b];
    s.start = st < 0 ? 0 : (st > a.ctx_cap ? a.ctx_cap : st);
    s.ctx = min(s.start + s.tokens, a.ctx_cap);
    s.tiles = s.tokens > 0 ? (s.ctx + kTK - 1) / kTK : 0;
    return s;
}

// Places of one unit of `tiles` tiles on the line: its start-up cost, then its tiles.
__device__ __forceinline__ int unit_span(int tiles) { return tiles > 0 ? kPieceCostTiles + tiles : 0; }

__device__ __forceinline__ int64_t scan_lanes(int64_t x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// The sequence whose units hold line place `pos`, searching from sequence b0 whose
// units start at `base` (wave-wide, 64 sequences per step); false past the end.
__device__ bool locate_tile(const MultiArgs &a, int64_t pos, int b0, int64_t base, int &b_out, int64_t &start_out) {
    const int lane = threadIdx.x & 63;
    for (; b0 < a.batch; b0 += 64) {
        const int bb = b0 + lane;
        const int sp = bb < a.batch ? unit_span(seq_info(a, bb).tiles) : 0;
        const int64_t incl = scan_lanes((int64_t)sp * a.hgroups, lane);
        const int64_t total = __shfl(incl, 63);
        if (pos < base + total) {
            const int l = __builtin_ctzll(__ballot(base + incl > pos));
            b_out = b0 + l;
            start_out = base + __shfl(incl, l) - (int64_t)__shfl(sp, l) * a.hgroups;
            return true;
        }
        base += total;
    }
    return false;
}

// Places per workgroup for a line of `total` places: spread over `target` workgroups
// (one round on the chip), within [kMultiMinTilesPerWorkgroup, kMultiMaxTilesPerWorkgroup].
__device__ __forceinline__ int per_for_line(const MultiArgs &a, int64_t total) {
    int64_t per = (total + a.target - 1) / a.target;
    per = per < kMultiMinTilesPerWorkgroup ? kMultiMinTilesPerWorkgroup : per;
    return (int)(per > kMultiMaxTilesPerWorkgroup ? kMultiMaxTilesPerWorkgroup : per);
}

// Places per workgroup of this call's line and the sequence whose units hold this
// workgroup's first place (sb: the line place of its first unit); false when the
// workgroup is past the line's end (wave-wide).  One pass over the sequences: the first
// 64 stay in registers for the search.
__device__ bool workgroup_range(const MultiArgs &a, int &per, int &b, int64_t &sb) {
    const int lane = threadIdx.x & 63;
    int64_t total = 0, incl0 = 0;
    int sp0 = 0;
    for (int b0 = 0; b0 < a.batch; b0 += 64) {
        const int bb = b0 + lane;
        const int sp = bb < a.batch ? unit_span(seq_info(a, bb).tiles) : 0;
        const int64_t incl = scan_lanes((int64_t)sp * a.hgroups, lane);
        if (b0 == 0) {
            sp0 = sp;
            incl0 = incl;
        }
        total += __shfl(incl, 63);
    }
    per = per_for_line(a, total);
    const int64_t r0 = (int64_t)blockIdx.x * per;
    const int64_t first = __shfl(incl0, 63);
    if (r0 < first) {
        const int l = __builtin_ctzll(__ballot(incl0 > r0));
        b = l;
        sb = __shfl(incl0, l) - (int64_t)__shfl(sp0, l) * a.hgroups;
        return true;
    }
    return locate_tile(a, r0, 64, first, b, sb);
}

__device__ __forceinline__ int page_of(const MultiArgs &a, int t) {
    return a.page_shift >= 0 ? (t >> a.page_shift) : t / a.page_size;
}

template <int D>
struct MultiTiling {
    static constexpr int TEAMS = D == 128 ? 2 : 1;
    static constexpr int NGRP = D == 128 ? 3 : 2;
};

// Gather the K and V rows of tokens 32*t .. 32*t + 31 (clamped to ctx - 1) of one
// KV head into an LDS stage through the piece's page ids; the waves split the slots.
// Nontemporal loads: each K/V row is read once per call (for all query columns of
// its KV head), from pools larger than the last-level cache.
template <int D, int NW>
__device__ __forceinline__ void issue_tile(const MultiArgs &a, uint16_t *k_tile, uint16_t *v_tile, const int *s_pg,
                                           int pg0, int t, int ctx, int64_t head_off, int wave, int lane) {
    constexpr int CH = D / 8;
    constexpr int NLD = kTK * CH / (64 * NW);
    const uint32_t kb = (uint32_t)(uintptr_t)(lds_void *)k_tile;
    const uint32_t vb = (uint32_t)(uintptr_t)(lds_void *)v_tile;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int slot = (i * NW + wave) * 64 + lane;
        const int row = slot / CH, pch = slot % CH;
        int tok = kTK * t + row;
        tok = tok < ctx ? tok : ctx - 1;
        const int pg = page_of(a, tok);
        const int64_t off = (int64_t)s_pg[pg - pg0] * a.page_stride + (int64_t)(tok - pg * a.page_size) * a.token_stride +
                            head_off;
        const uint16_t *ksrc = a.k_pool + off + 8 * (pch ^ attend_k_swz(row));
        const uint16_t *vsrc = a.v_pool + off + 8 * (pch ^ attend_v_swz(row));
        const uint32_t mk = __builtin_amdgcn_readfirstlane(kb + (i * NW + wave) * 1024);
        const uint32_t mv = __builtin_amdgcn_readfirstlane(vb + (i * NW + wave) * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(mk), "v"(ksrc) : "memory");
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(mv), "v"(vsrc) : "memory");
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

// One piece: tiles [ta, tb) of sequence b for workgroup head group hg, written as
// partial `split` of its columns.
template <int D, int NWV, bool BF16>
__device__ __forceinline__ void multi_piece(const MultiArgs &a, uint16_t *kv_lds, int *s_pg, int b, const SeqInfo &si,
                                            int hg, int ta, int tb, int split) {
    constexpr int TEAMS = MultiTiling<D>::TEAMS;
    constexpr int NGRP = MultiTiling<D>::NGRP;
    constexpr int NSTAGE = TEAMS * NGRP;
    constexpr int NW = TEAMS * NWV;
    constexpr int TILE = kTK * D;
    constexpr int KSTEPS = D / 32;
    constexpr int DBLK = D / 16;
    constexpr int NLD = kTK * (D / 8) / (64 * NW);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int team = wave / NWV, cw = wave % NWV;
    const int kh = hg / a.qgroups, qg = hg % a.qgroups;
    const int64_t head_off = (int64_t)kh * a.head_stride;

    // page ids of the piece (entries past the context are never read)
    const int tok0 = kTK * ta, tok1 = min(kTK * tb, si.ctx);
    const int pg0 = page_of(a, tok0);
    const int npg = page_of(a, tok1 - 1) - pg0 + 1;
    for (int i = threadIdx.x; i < npg; i += blockDim.x) {
        int page = a.page_table[(int64_t)b * a.max_pages + pg0 + i];
        s_pg[i] = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
    }
    __syncthreads();

    // first ring of tiles in flight while Q is read
#pragma unroll
    for (int k = 0; k < TEAMS * (NGRP - 1); ++k) {
        const int t = ta + k;
        if (t < tb) {
            uint16_t *st = kv_lds + k * 2 * TILE;
            issue_tile<D, NW>(a, st, st + TILE, s_pg, pg0, t, si.ctx, head_off, wave, lane);
        }
    }

    // query column of this lane: (head of the group, token)
    const int slot = lane & 15, g4 = lane >> 4;
    const int col = 16 * cw + slot;
    const int hh = col / a.max_tokens, qi = col % a.max_tokens;
    const bool col_ok = col < a.ncols && qi < si.tokens;
    const int head = kh * a.group + qg * a.heads_per_wg + (col < a.ncols ? hh : 0);
    const int limit = min(si.start + qi + 1, si.ctx);          // keys t < limit are visible
    const int first_limit = min(si.start + 1, si.ctx);         // the first token's frontier

    // Q^T (scaled by scale * log2 e) as the B operand: column = lane % 16, k = 32*ks + 8*(lane/16) + e;
    // bf16 keeps 8 significant bits, so the rest of Q rides in a second operand
    uint4v qf[KSTEPS], qlo[KSTEPS];
    {
        const float *qp = a.q + b * a.q_bs + (int64_t)(col_ok ? qi : 0) * a.q_ts + (int64_t)head * a.q_hs + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const float4v x0 = *reinterpret_cast<const float4v *>(qp + 32 * ks);
            const float4v x1 = *reinterpret_cast<const float4v *>(qp + 32 * ks + 4);
            float x[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = col_ok ? x0[e] * a.score_scale : 0.f;
                x[4 + e] = col_ok ? x1[e] * a.score_scale : 0.f;
            }
            uint16_t h[8], r[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                h[e] = to_kv16<BF16>(x[e]);
                r[e] = to_kv16<BF16>(x[e] - from_kv16<BF16>(h[e]));
            }
            qf[ks] = uint4v{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
            qlo[ks] = uint4v{pack2(r[0], r[1]), pack2(r[2], r[3]), pack2(r[4], r[5]), pack2(r[6], r[7])};
        }
    }

    float4v acc[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) acc[db] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const int ngroups = (tb - ta + TEAMS - 1) / TEAMS;
    int gstage = 0;  // first stage of the group in use
    for (int k = 0; k < ngroups; ++k) {
        // tiles issued after group k: up to the end of group k + NGRP - 2
        const int issued_end = min(tb, ta + TEAMS * (k + NGRP - 1));
        const int after = max(0, issued_end - (ta + TEAMS * (k + 1)));
        attend_wait_tiles<2 * NLD>(after);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // every wave's part of group k is in
        {
            // group k + NGRP - 1 goes into the stages of group k - 1: every wave is past it
            const int sn = gstage == 0 ? NSTAGE - TEAMS : gstage - TEAMS;
#pragma unroll
            for (int e = 0; e < TEAMS; ++e) {
                const int tn = ta + TEAMS * (k + NGRP - 1) + e;
                if (tn < tb) {
                    uint16_t *st = kv_lds + (sn + e) * 2 * TILE;
                    issue_tile<D, NW>(a, st, st + TILE, s_pg, pg0, tn, si.ctx, head_off, wave, lane);
                }
            }
        }
        const int t = ta + TEAMS * k + team;
        if (t < tb) {
            const uint16_t *k_tile = kv_lds + (gstage + team) * 2 * TILE;
            attend_tile<D, kTK, BF16, BF16>(k_tile, k_tile + TILE, qf, qlo, 1.f, kTK * (t + 1) > first_limit,
                                            kTK * t, limit, acc, m_run, l_run, lane);
        }
        gstage = gstage + TEAMS == NSTAGE ? 0 : gstage + TEAMS;
    }

    if constexpr (TEAMS == 2) attend_merge_teams<D, NWV>(kv_lds, team, cw, lane, acc, m_run, l_run);

    if (team == 0 && col_ok) {
        const int64_t u = (((int64_t)b * a.max_tokens + qi) * a.n_heads + head) * a.max_splits + split;
        float *dst = a.part + u * D + 4 * g4;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) *reinterpret_cast<float4v *>(dst + 16 * db) = acc[db];
        if (g4 == 0) a.ml[u] = make_float2(m_run, l_run);
    }
    __syncthreads();  // the next piece reuses the stages and the page ids
}

template <int D, int NWV, bool BF16>
__global__ __launch_bounds__(64 * NWV * MultiTiling<D>::TEAMS) void multi_partial_kernel(MultiArgs a) {
    constexpr int TEAMS = MultiTiling<D>::TEAMS;
    constexpr int NSTAGE = TEAMS * MultiTiling<D>::NGRP;
    constexpr int DBLK = D / 16;
    constexpr int TILE = kTK * D;
    static_assert((kTK * (D / 8)) % (64 * TEAMS * NWV) == 0, "tile slots must split evenly over the waves");
    static_assert(TEAMS * (MultiTiling<D>::NGRP - 1) <= 6 &&
                      TEAMS * (MultiTiling<D>::NGRP - 1) * 2 * (kTK * (D / 8) / (64 * TEAMS * NWV)) <= 63,
                  "vmcnt immediates");
    static_assert(TEAMS == 1 || NWV * (DBLK * 64 * 16 + 64 * 8) <= NSTAGE * 2 * TILE * 2, "team exchange fits");
    __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[NSTAGE * 2 * TILE];  // [stage][K, V]
    __shared__ int s_pg[kPgCap];

    // line places [r0, r1) of this workgroup, cut at unit boundaries into pieces; a unit
    // is its start-up places, then its tiles [rs, u1)
    int per, b;
    int64_t sb;
    if (!workgroup_range(a, per, b, sb)) return;
    const int64_t r0 = (int64_t)blockIdx.x * per, r1 = r0 + per;
    SeqInfo si = seq_info(a, b);
    int span = unit_span(si.tiles);
    int64_t pos = r0;
    for (;;) {
        const int hg = (int)((pos - sb) / span);
        const int64_t u0 = sb + (int64_t)hg * span, rs = u0 + kPieceCostTiles, u1 = u0 + span;
        const int64_t e = u1 < r1 ? u1 : r1;
        const int64_t ps = pos > rs ? pos : rs;
        if (ps < e) {
            const int split = blockIdx.x - (int)(rs / per);
            if (split == 0 && threadIdx.x == 0)
                a.npiece[(int64_t)b * a.hgroups + hg] = (int)((u1 - 1) / per - rs / per + 1);
            multi_piece<D, NWV, BF16>(a, kv_lds, s_pg, b, si, hg, (int)(ps - rs), (int)(e - rs), split);
        }
        pos = e;
        if (pos >= r1) break;
        const int64_t seq_end = sb + (int64_t)span * a.hgroups;
        if (pos >= seq_end) {
            if (!locate_tile(a, pos, b + 1, seq_end, b, sb)) break;
            si = seq_info(a, b);
            span = unit_span(si.tiles);
        }
    }
}

// Half a wave per (sequence, token, query head) row: O = sum_s 2^(m_s - M) O_s / sum_s
// 2^(m_s - M) l_s over the pieces of its unit; rows past the sequence's query length are
// not written.  Every load the merge needs (the sequence's lengths, the unit's piece
// count, the first 32 (m, l) and the first NP slices) is issued at once, whatever the
// count turns out to be, so a row of at most NP pieces costs one memory round trip;
// slots past the count are never used (they may hold anything).
template <int D>
__global__ __launch_bounds__(256) void multi_merge_kernel(MultiArgs a) {
    constexpr int PER = D / 32;  // floats per lane
    constexpr int NV = PER / 4;  // float4 per lane and piece
    constexpr int NP = 4;        // pieces loaded up front
    const int lane = threadIdx.x & 63, l32 = lane & 31, hbase = lane & 32;
    const int64_t rows = (int64_t)a.batch * a.max_tokens * a.n_heads;
    const int64_t wrow = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2;
    if (wrow >= rows) return;  // the whole wave
    const bool valid = wrow + (lane >> 5) < rows;
    const int64_t row = valid ? wrow + (lane >> 5) : rows - 1;
    const int head = (int)(row % a.n_heads);
    const int qi = (int)((row / a.n_heads) % a.max_tokens);
    const int b = (int)(row / ((int64_t)a.n_heads * a.max_tokens));
    const int hg = (head / a.group) * a.qgroups + (head % a.group) / a.heads_per_wg;

    const SeqInfo si = seq_info(a, b);
    const int np_raw = a.npiece[(int64_t)b * a.hgroups + hg];
    const float2 *mlr = a.ml + row * a.max_splits;
    const float *pr = a.part + row * a.max_splits * D + l32 * PER;
    const float2 my0 = l32 < a.max_splits ? mlr[l32] : make_float2(-INFINITY, 0.f);
    float4v v0[NP][NV];
#pragma unroll
    for (int u = 0; u < NP; ++u)
#pragma unroll
        for (int i = 0; i < NV; ++i)
            v0[u][i] = u < a.max_splits ? *reinterpret_cast<const float4v *>(pr + (int64_t)u * D + 4 * i)
                                        : float4v{0.f, 0.f, 0.f, 0.f};
    // a unit without tiles (no visible key) has no pieces and a row of zeros
    const int nsplit = si.tiles == 0 ? 0 : min(max(np_raw, 0), a.max_splits);

    float mmax = l32 < nsplit ? my0.x : -INFINITY;
    for (int s = 32 + l32; s < nsplit; s += 32) mmax = fmaxf(mmax, mlr[s].x);
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) mmax = fmaxf(mmax, __shfl_xor(mmax, off));
    float4v o[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) o[i] = float4v{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    if (mmax != -INFINITY) {
        for (int s0 = 0; s0 < nsplit; s0 += 32) {
            const bool mine = s0 + l32 < nsplit;
            const float2 m2 = s0 == 0 ? my0 : (mine ? mlr[s0 + l32] : make_float2(-INFINITY, 0.f));
            const float w = mine && m2.x != -INFINITY ? exp2f(m2.x - mmax) : 0.f;
            float lw = w > 0.f ? w * m2.y : 0.f;
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) lw += __shfl_xor(lw, off);
            lsum += lw;
            const int n = min(32, nsplit - s0);
            for (int j = 0; j < n; j += NP) {
                if (s0 > 0 || j > 0) {  // past the slices loaded up front: load the next NP into v0
#pragma unroll
                    for (int u = 0; u < NP; ++u)
#pragma unroll
                        for (int i = 0; i < NV; ++i)
                            v0[u][i] = j + u < n ? *reinterpret_cast<const float4v *>(
                                                       pr + (int64_t)(s0 + j + u) * D + 4 * i)
                                                 : float4v{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int u = 0; u < NP; ++u) {
                    const float wj = __shfl(w, hbase | ((j + u) & 31));
                    if (j + u < n) {
#pragma unroll
                        for (int i = 0; i < NV; ++i) o[i] += wj * v0[u][i];
                    }
                }
            }
        }
    }
    if (!valid || qi >= si.tokens) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float *orow = a.o + b * a.o_bs + (int64_t)qi * a.o_ts + (int64_t)head * a.o_hs + l32 * PER;
#pragma unroll
    for (int i = 0; i < NV; ++i) *reinterpret_cast<float4v *>(orow + 4 * i) = o[i] * inv;
}

template <int D, int NWV, bool BF16>
hipError_t launch_typed(const MultiArgs &a, int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL((multi_partial_kernel<D, NWV, BF16>), dim3((unsigned)grid),
                       dim3(64 * NWV * MultiTiling<D>::TEAMS), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t rows = (int64_t)a.batch * a.max_tokens * a.n_heads;
    hipLaunchKernelGGL((multi_merge_kernel<D>), dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_waves(const MultiArgs &a, int64_t grid, hipStream_t stream) {
    const int waves = (a.ncols + 15) / 16;
    if (waves <= 1) return launch_typed<D, 1, BF16>(a, grid, stream);
    if (waves <= 2) return launch_typed<D, 2, BF16>(a, grid, stream);
    return launch_typed<D, 4, BF16>(a, grid, stream);
}

}  // namespace

// One workgroup per CU of the current device (the LDS ring takes most of a CU's LDS).
int multi_target_workgroups() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        return kMultiDefaultWorkgroups;
    return cus;
}

int plan_paged_prefill(const attn_paged_prefill_params *p, MultiPlan *plan) {
    plan->group = p->n_heads / p->n_kv_heads;
    int gw = 1;  // query heads per workgroup: the largest divisor of the group whose tokens fit 64 columns
    for (int c = 1; c <= plan->group && c * p->max_tokens <= 64; ++c)
        if (plan->group % c == 0) gw = c;
    plan->heads_per_wg = gw;
    plan->qgroups = plan->group / gw;
    plan->hgroups = p->n_kv_heads * plan->qgroups;
    int cap = p->max_context;
    const int64_t table_cap = (int64_t)p->max_pages_per_seq * p->page_size;
    if (table_cap < cap) cap = (int)table_cap;
    if (cap < 0) cap = 0;
    plan->ctx_cap = cap;
    const int64_t tiles_max = ((int64_t)cap + kTK - 1) / kTK;
    // a unit of T tiles overlaps at most ceil(T / per) + 1 workgroup ranges
    plan->max_splits = (int)((tiles_max + kMultiMinTilesPerWorkgroup - 1) / kMultiMinTilesPerWorkgroup + 1);
    plan->target = multi_target_workgroups();
    // enough workgroups for the longest line at the most places per workgroup
    const int64_t line = (int64_t)p->batch * plan->hgroups * (tiles_max + kPieceCostTiles);
    const int64_t need = (line + kMultiMaxTilesPerWorkgroup - 1) / kMultiMaxTilesPerWorkgroup;
    plan->grid = need > plan->target ? need : plan->target;
    const size_t rows = (size_t)p->batch * p->max_tokens * p->n_heads;
    plan->ml_offset = 0;
    plan->ml_bytes = rows * plan->max_splits * sizeof(float2);
    plan->part_offset = (plan->ml_bytes + 255) & ~(size_t)255;
    plan->part_bytes = rows * plan->max_splits * p->head_dim * sizeof(float);
    plan->npiece_offset = (plan->part_offset + plan->part_bytes + 255) & ~(size_t)255;
    plan->npiece_bytes = (size_t)p->batch * plan->hgroups * sizeof(int32_t);
    plan->workspace_bytes = plan->npiece_offset + plan->npiece_bytes;
    return ATTN_OK;
}

hipError_t launch_paged_prefill(const attn_paged_prefill_params *p, const MultiPlan *plan, const float *q,
                                const void *k_pool, const void *v_pool, const int32_t *page_table,
                                const int32_t *query_lens, const int32_t *position_starts, float *o, void *ws,
                                hipStream_t stream) {
    MultiArgs a;
    a.q = q;
    a.k_pool = (const uint16_t *)k_pool;
    a.v_pool = (const uint16_t *)v_pool;
    a.page_table = page_table;
    a.query_lens = query_lens;
    a.position_starts = position_starts;
    a.o = o;
    a.ml = (float2 *)((uint8_t *)ws + plan->ml_offset);
    a.part = (float *)((uint8_t *)ws + plan->part_offset);
    a.npiece = (int32_t *)((uint8_t *)ws + plan->npiece_offset);
    a.q_bs = p->q_bs;
    a.q_ts = p->q_ts;
    a.q_hs = p->q_hs;
    a.o_bs = p->o_bs;
    a.o_ts = p->o_ts;
    a.o_hs = p->o_hs;
    a.page_stride = p->kv_page_stride;
    a.token_stride = p->kv_token_stride;
    a.head_stride = p->kv_head_stride;
    a.batch = p->batch;
    a.n_heads = p->n_heads;
    a.group = plan->group;
    a.heads_per_wg = plan->heads_per_wg;
    a.qgroups = plan->qgroups;
    a.hgroups = plan->hgroups;
    a.max_tokens = p->max_tokens;
    a.ncols = plan->heads_per_wg * p->max_tokens;
    a.page_size = p->page_size;
    a.max_pages = p->max_pages_per_seq;
    a.num_pages = p->num_pages;
    a.ctx_cap = plan->ctx_cap;
    a.target = plan->target;
    a.max_splits = plan->max_splits;
    a.score_scale = p->scale * kLog2e;
    int shift = -1;
    for (int k = 0; k < 31; ++k)
        if ((1 << k) == p->page_size) shift = k;
    a.page_shift = shift;
    const bool bf16 = p->kv_dtype == ATTN_BF16;
    switch (p->head_dim) {
    case 128: return bf16 ? launch_waves<128, true>(a, plan->grid, stream) : launch_waves<128, false>(a, plan->grid, stream);
    case 256: return bf16 ? launch_waves<256, true>(a, plan->grid, stream) : launch_waves<256, false>(a, plan->grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
