// narrow.hip -- prefill attention at head_dim 128/256 with two waves per SIMD.
//
// What is computed is what prefill.hip computes (mlx-native 0.18.0,
// src/ops/flash_attn_prefill_tensor.rs, module header): O = softmax(scale Q K^T +
// mask) V with an online softmax over 64-row KV tiles.  This file holds the
// kernel for 128-slot workgroups at head_dim <= 256.  It is compiled with MFMA
// accumulators in ordinary VGPRs (-mllvm -amdgpu-mfma-vgpr-form), so that a
// wave's whole budget of 256 registers is one pool: O (64 registers at head_dim
// 256), the scores and Q share it.
#include "prefill_common.h"

namespace attn {
namespace {

// narrow_kernel: head_dim 128/256 with 16 query slots per wave and two waves per
// SIMD.  A wave's O^T (16 slots x D) is D/16 v_mfma_f32_16x16x32 accumulator blocks
// (64 AGPRs at head_dim 256) and its Q fragment 32 VGPRs, so eight waves of a
// 128-slot workgroup fit the register file two to a SIMD: while one wave of a
// SIMD runs its softmax, waits on a barrier or issues loads, the other one's
// MFMAs keep the matrix core busy.  S^T = K Q^T per 16-key block (lane: query
// slot lane%16, keys 4*(lane/16) + 0..3 of the block); P^T goes from those
// accumulators into the B operand of O^T += V^T P^T with the 32 keys of a half
// stage ordered {4g..4g+3, 16+4g..16+4g+3} in lane group g, and V^T comes from
// ds_read_b64_tr_b16 in the same key order.  Stages, tile codes, the row-block
// pairing, KV splits, the status block and the workspace are those of
// prefill_kernel.
template <int D, int NW, bool BF16, int MASK, bool QSPLIT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void narrow_kernel(
    PrefillArgs a) {
    constexpr bool HAS_MASK = MASK != 0;
    constexpr bool MBF16 = MASK == 2;
    constexpr int BK = 64;                 // keys per stage: one tile code
    constexpr int KSTEPS = D / 32;         // k-steps of S^T
    constexpr int DBLK = D / 16;           // 16-column O blocks
    constexpr int STAGE_ELEMS = BK * D;
    using KS = TileStream<D, NW, BK, kSwzK>;
    using VS = TileStream<D, NW, BK, kSwzV16>;
    static_assert(KS::NLD == VS::NLD, "K and V stream alike");
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2 * STAGE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2 * STAGE_ELEMS];
    constexpr int MI = 2;                  // mask DMA instructions per wave per stage (16 rows x 64 keys)
    __shared__ __attribute__((aligned(1024))) uint4v m_lds[HAS_MASK ? 2 * NW * MI * 64 : 1];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j16 = lane & 15;   // query slot column of the wave
    const int g4 = lane >> 4;    // lane group: k chunk of an operand, row group of an accumulator
    if constexpr (!HAS_MASK) {
        if (blockIdx.x == 0 && threadIdx.x < kStatusWords) a.status[threadIdx.x] = 0u;
    }

    int lin = blockIdx.x;
    const int hg = lin % a.head_groups;
    lin /= a.head_groups;
    const int idx = lin % a.row_blocks;
    lin /= a.row_blocks;
    const int split = lin % a.splits;
    const int b = lin / a.splits;
    const int h0 = hg * a.heads_per_wg;
    const int kvh = h0 / a.group;
    const int n_stages = (a.kv_len + BK - 1) / BK;
    const int split_begin = split * a.tiles_per_split;
    const int split_end = min(split_begin + a.tiles_per_split, n_stages);

    // tasks: as in prefill_kernel (heavy row blocks first; with pairing, heavy block hi
    // and light block lo of a pair shared by two workgroups with a cut in hi)
    const PrefillTasks tasks = prefill_tasks<1, HAS_MASK>(a, b, hg, idx, split_begin, split_end, n_stages, lane);
    const int rb0 = tasks.rb0, beg0 = tasks.beg0, end0 = tasks.end0, side0 = tasks.side0;
    const int rb1 = tasks.rb1, beg1 = tasks.beg1, end1 = tasks.end1, ntask = tasks.ntask, pair = tasks.pair;

    // lane offsets of the MFMA operand reads (a few per lane, the rest immediates)
    //  K (A operand of S^T): key block kb, k-step ks = 4q + r reads row 16*kb + j16, logical
    //    chunk 4*ks + g4, stored at chunk ^ j16: k_off[r] + 256*q + kb*32*D
    uint32_t k_off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) k_off[r] = (uint32_t)((j16 * D + 8 * ((4 * r + g4) ^ j16)) * 2);
    //  V^T (A operand of O^T, transposing reads): half h, block db; lane j16 of group g4
    //    points at row 32h + 4*g4 + j16/4 (and +16), column 16*db + 4*(j16&3); the chunk
    //    2*db + (j16&3)/2 is stored at chunk ^ 2*(row&7), a lane constant:
    //    v_off[db&7] + 256*(db>>3) + h*64*D (+32*D for the second read)
    uint32_t v_off[DBLK < 8 ? DBLK : 8];
    {
        const int vrow = 4 * g4 + (j16 >> 2);
        const int swz = 2 * (vrow & 7);
        const int c0 = (j16 & 3) >> 1;
#pragma unroll
        for (int q = 0; q < (DBLK < 8 ? DBLK : 8); ++q)
            v_off[q] = (uint32_t)((vrow * D + 4 * (j16 & 1) + 8 * ((2 * q + c0) ^ swz)) * 2);
    }
    //  mask (16 rows x 64 keys per wave and stage): chunk c (8 keys) of row r is stored at
    //    c ^ ((r >> 1) & 7); key block kb of this lane is chunk 2*kb + g4/2, half g4&1
    uint32_t m_off[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        m_off[kb] = (uint32_t)((j16 * 8 + ((2 * kb + (g4 >> 1)) ^ ((j16 >> 1) & 7))) * 16 + 8 * (g4 & 1));

    for (int task = 0; task < ntask; ++task) {
    const int rb = task == 0 ? rb0 : rb1;
    const int st_begin = task == 0 ? beg0 : beg1;
    const int st_end = task == 0 ? end0 : end1;
    const int side = task == 0 ? side0 : -1;

    const int slot = wave * 16 + j16;
    const int head = h0 + slot / a.rows_per_wg;
    const int row = rb * a.rows_per_wg + slot % a.rows_per_wg;
    const bool row_ok = row < a.rows;
    const int row_c = row_ok ? row : a.rows - 1;

    const uint16_t *mrow = nullptr;
    // mask DMA: instruction n, lane i fills slot 64n + i of the wave's region, i.e. row
    // 8n + i/8 of the wave's 16, stored chunk i%8
    const uint16_t *mdma[MI];
    if constexpr (HAS_MASK) {
        mrow = (const uint16_t *)a.mask + b * a.m_bs + head * a.m_hs + (int64_t)row_c * a.m_rs;
#pragma unroll
        for (int n = 0; n < MI; ++n) {
            const int r16 = 8 * n + (lane >> 3);
            const int sl = wave * 16 + r16;
            const int mh = h0 + sl / a.rows_per_wg;
            int mr_ = rb * a.rows_per_wg + sl % a.rows_per_wg;
            mr_ = mr_ < a.rows ? mr_ : a.rows - 1;
            const int c = (lane & 7) ^ ((r16 >> 1) & 7);
            mdma[n] = (const uint16_t *)a.mask + b * a.m_bs + mh * a.m_hs + (int64_t)mr_ * a.m_rs + 8 * c;
        }
    }

    float4v acc_o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) acc_o[db] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_bs + kvh * a.k_hs;
    const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_bs + kvh * a.v_hs;
    const_u32 *blk_row = nullptr;
    if constexpr (HAS_MASK) {
        const int bh = a.blk_heads == 1 ? 0 : hg;
        blk_row = (const_u32 *)(a.blk + (((int64_t)b * a.blk_heads + bh) * a.row_blocks + rb) * a.blk_stride);
    }
    auto stage_code = [&](int st_) -> int {
        if constexpr (HAS_MASK) return (int)((blk_row[st_ >> 2] >> (8 * (st_ & 3))) & 0xffu);
        else return TILE_OPEN;
    };
    auto next_stage = [&](int from) {
        int st_ = from;
        while (st_ < st_end && stage_code(st_) == TILE_SKIP) ++st_;
        return st_ < st_end ? st_ : st_end;
    };
    auto mask_in_lds = [&](int st_) { return a.mask_dma && st_ * BK + BK <= a.kv_len; };
    auto issue_mask_one = [&](int st_, int bufi, int n) __attribute__((always_inline)) {
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(
            (uint32_t)(uintptr_t)(lds_void *)(m_lds + ((bufi * NW + wave) * MI + n) * 64));
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(mdma[n] + st_ * BK)
                     : "memory");
    };

    KS kstream;
    VS vstream;
    kstream.init(lane, wave, a.k_rs);
    vstream.init(lane, wave, a.v_rs);

    int st = next_stage(st_begin);
    int buf = 0;
    auto issue_first_stage = [&]() {
        if (st < st_end) {
            if (HAS_MASK && stage_code(st) == TILE_MASKED && mask_in_lds(st)) {
#pragma unroll
                for (int n = 0; n < MI; ++n) issue_mask_one(st, 0, n);
            }
            const bool full = st * BK + BK <= a.kv_len;
            kstream.issue(k_lds, kbase, a.k_rs, st * BK, a.kv_len, wave, full);
            vstream.issue(v_lds, vbase, a.v_rs, st * BK, a.kv_len, wave, full);
        }
    };

    // ---- Q^T fragment (B operand of S^T): column j16, k = 32*ks + 8*g4 + i; f32 Q is
    // scaled by scale*log2(e) before rounding, except bf16 Q against bf16 K/V (used as given)
    constexpr bool PRESCALE = !BF16 || QSPLIT;
    const float q_scale = PRESCALE ? a.score_scale : 1.f;
    const float post_scale = PRESCALE ? 1.f : a.score_scale;
    uint4v qf[KSTEPS];
    uint4v qlo[QSPLIT ? KSTEPS : 1];
    if (!a.q_bf16) {
        const float *qrow = reinterpret_cast<const float *>(a.q) + b * a.q_bs + (int64_t)row_c * a.q_rs +
                            (int64_t)head * a.q_hs + 8 * g4;
        float4v qraw[KSTEPS][2];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            qraw[ks][0] = *reinterpret_cast<const float4v *>(qrow + 32 * ks);
            qraw[ks][1] = *reinterpret_cast<const float4v *>(qrow + 32 * ks + 4);
        }
        issue_first_stage();  // shares the round trip of the Q loads
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const float4v x0 = qraw[ks][0] * q_scale;
            const float4v x1 = qraw[ks][1] * q_scale;
            uint4v cv;
            cv[0] = pack2(to_kv16<BF16>(x0[0]), to_kv16<BF16>(x0[1]));
            cv[1] = pack2(to_kv16<BF16>(x0[2]), to_kv16<BF16>(x0[3]));
            cv[2] = pack2(to_kv16<BF16>(x1[0]), to_kv16<BF16>(x1[1]));
            cv[3] = pack2(to_kv16<BF16>(x1[2]), to_kv16<BF16>(x1[3]));
            qf[ks] = row_ok ? cv : uint4v{0u, 0u, 0u, 0u};
            if constexpr (QSPLIT) {
                float rest[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rest[e] = x0[e] - bf16_bits_to_f32((uint16_t)(cv[e / 2] >> (16 * (e & 1))));
                    rest[4 + e] = x1[e] - bf16_bits_to_f32((uint16_t)(cv[2 + e / 2] >> (16 * (e & 1))));
                }
                const uint4v lo = uint4v{pack2(f32_to_bf16_rne(rest[0]), f32_to_bf16_rne(rest[1])),
                                         pack2(f32_to_bf16_rne(rest[2]), f32_to_bf16_rne(rest[3])),
                                         pack2(f32_to_bf16_rne(rest[4]), f32_to_bf16_rne(rest[5])),
                                         pack2(f32_to_bf16_rne(rest[6]), f32_to_bf16_rne(rest[7]))};
                qlo[ks] = row_ok ? lo : uint4v{0u, 0u, 0u, 0u};
            }
        }
    } else {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) + b * a.q_bs + (int64_t)row_c * a.q_rs +
                               (int64_t)head * a.q_hs + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const uint4v *>(qrow + 32 * ks);
        issue_first_stage();
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if constexpr (!BF16) {
                uint4v cv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_bits_to_f32((uint16_t)(qf[ks][e] & 0xffffu)) * q_scale;
                    const float hi = bf16_bits_to_f32((uint16_t)(qf[ks][e] >> 16)) * q_scale;
                    cv[e] = pack2(to_kv16<false>(lo), to_kv16<false>(hi));
                }
                qf[ks] = cv;
            }
            if (!row_ok) qf[ks] = uint4v{0u, 0u, 0u, 0u};
            if constexpr (QSPLIT) qlo[ks] = uint4v{0u, 0u, 0u, 0u};
        }
    }

    while (st < st_end) {
        const int code = stage_code(st);
        const int nxt = next_stage(st + 1);
        const int key0 = st * BK;
        const bool full_stage = key0 + BK <= a.kv_len;
        const bool use_mask = HAS_MASK && code == TILE_MASKED;

        wait_all_barrier();  // K, V and mask of this stage landed (all requested one stage ago)

        // stage nxt into the other buffers: a full stage one instruction at a time between
        // the S MFMAs, a ragged or widely strided one at once here
        const bool nfull = nxt < st_end && nxt * BK + BK <= a.kv_len && a.k_rs < kOff32Stride &&
                           a.v_rs < kOff32Stride;
        const bool nmask = HAS_MASK && nxt < st_end && stage_code(nxt) == TILE_MASKED && mask_in_lds(nxt);
        if (nxt < st_end && !nfull) {
            if (nmask) {
#pragma unroll
                for (int n = 0; n < MI; ++n) issue_mask_one(nxt, buf ^ 1, n);
            }
            kstream.issue(k_lds + (buf ^ 1) * STAGE_ELEMS, kbase, a.k_rs, nxt * BK, a.kv_len, wave, false);
            vstream.issue(v_lds + (buf ^ 1) * STAGE_ELEMS, vbase, a.v_rs, nxt * BK, a.kv_len, wave, false);
        }
        const char *kst = KS::stage_ptr(kbase, a.k_rs, nxt * BK, wave);
        const char *vst = VS::stage_ptr(vbase, a.v_rs, nxt * BK, wave);
        uint16_t *kdst = k_lds + (buf ^ 1) * STAGE_ELEMS;
        uint16_t *vdst = v_lds + (buf ^ 1) * STAGE_ELEMS;
        // instruction n of the next stage: mask chunks first, then K and V alternately
        constexpr int NDMA = (HAS_MASK ? MI : 0) + 2 * KS::NLD;
        auto dma_one = [&](auto n_c) __attribute__((always_inline)) {
            constexpr int n = decltype(n_c)::value;
            if constexpr (HAS_MASK && n < MI) {
                if (nmask) issue_mask_one(nxt, buf ^ 1, n);
            } else {
                constexpr int jj = n - (HAS_MASK ? MI : 0);
                if constexpr (jj % 2 == 0) kstream.issue_one(kdst, kst, a.k_rs, jj / 2, wave);
                else vstream.issue_one(vdst, vst, a.v_rs, jj / 2, wave);
            }
        };
        const char *kt = reinterpret_cast<const char *>(k_lds + buf * STAGE_ELEMS);
        const char *vt = reinterpret_cast<const char *>(v_lds + buf * STAGE_ELEMS);

        // ---- S^T (64 keys x 16 slots): step i is k-step i/4 of key block i%4
        float4v s[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[kb] = float4v{0.f, 0.f, 0.f, 0.f};
        lds_pipeline<4 * KSTEPS, kLdsAhead, uint4v>(
            [&](int i) __attribute__((always_inline)) {
                const int kb = i % 4, ks = i / 4;
                return *reinterpret_cast<const uint4v *>(kt + k_off[ks & 3] + (ks >> 2) * 256 + kb * 32 * D);
            },
            [&](int i, const uint4v &kf) __attribute__((always_inline)) {
                s[i % 4] = mfma16<BF16>(kf, qf[i / 4], s[i % 4]);
                if constexpr (QSPLIT) s[i % 4] = mfma16<BF16>(kf, qlo[i / 4], s[i % 4]);
                if (nfull) {
                    static_for<NDMA>([&](auto n_c) __attribute__((always_inline)) {
                        if (i == (decltype(n_c)::value * 4 * KSTEPS) / NDMA) dma_one(n_c);
                    });
                }
            });

        // ---- scale and mask (log2 units); lane holds keys key0 + 16*kb + 4*g4 + e of slot j16
        if (use_mask) {
            uint2 mr[4];
            if (mask_in_lds(st)) {
                const char *mb = reinterpret_cast<const char *>(m_lds + (buf * NW + wave) * MI * 64);
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) mr[kb] = *reinterpret_cast<const uint2 *>(mb + m_off[kb]);
            } else {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const int kf = key0 + 16 * kb + 4 * g4;
                    uint16_t m16[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) m16[e] = mrow[min(kf + e, a.kv_len - 1)];
                    mr[kb] = make_uint2(pack2(m16[0], m16[1]), pack2(m16[2], m16[3]));
                }
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t word = e < 2 ? mr[kb].x : mr[kb].y;
                    const uint16_t m16 = (uint16_t)(word >> (16 * (e & 1)));
                    const float mv = MBF16 ? bf16_bits_to_f32(m16) : f16_bits_to_f32(m16);
                    s[kb][e] = PRESCALE ? fmaf(mv, kLog2e, s[kb][e]) : fmaf(s[kb][e], post_scale, mv * kLog2e);
                }
        } else if constexpr (!PRESCALE) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) s[kb] *= post_scale;
        }
        if (!full_stage) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (key0 + 16 * kb + 4 * g4 + e >= a.kv_len) s[kb][e] = -INFINITY;
        }

        // ---- online softmax for slot j16 (16 keys here, the rest in lanes ^16, ^32, ^48)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[kb][e]);
        mx = max_over_rows(mx);
        const bool grow = mx > m_run + kRescaleThreshold;  // also true for the first visible key
        const float m_new = grow ? mx : m_run;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        float rowsum = 0.f;
        // P^T for half h: k slot i <-> key 32h + 4*g4 + i (i < 4), 32h + 16 + 4*g4 + i - 4 (i >= 4)
        uint4v pb[2];
        uint4v pl[BF16 ? 2 : 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4v &sv = s[2 * h + (i >> 1)];
                const float p0 = __builtin_amdgcn_exp2f(sv[2 * (i & 1)] - m_use);
                const float p1 = __builtin_amdgcn_exp2f(sv[2 * (i & 1) + 1] - m_use);
                uint32_t hi, lo;
                if constexpr (BF16) {
                    pack_p_bf16(p0, p1, hi, lo, rowsum);
                    pl[h][i] = lo;
                } else {
                    hi = pack_p_f16(p0, p1, rowsum);
                }
                pb[h][i] = hi;
            }
        }
        rowsum = sum_over_rows(rowsum);
        l_run = l_run * alpha + rowsum;
        m_run = m_new;
        if (__ballot(grow)) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db) acc_o[db] *= alpha;
        }

        // ---- O^T[d][slot] += V^T[d][key] P^T[key][slot]; step i: half i / DBLK into block i % DBLK
        lds_pipeline<2 * DBLK, kLdsAhead, uint4v>(
            [&](int i) __attribute__((always_inline)) {
                const int h = i / DBLK, db = i % DBLK;
                const char *p0 = vt + v_off[db & 7] + 256 * (db >> 3) + h * 64 * D;
                return read_tr16_pair(reinterpret_cast<const uint16_t *>(p0),
                                      reinterpret_cast<const uint16_t *>(p0 + 32 * D));
            },
            [&](int i, const uint4v &vf) __attribute__((always_inline)) {
                acc_o[i % DBLK] = mfma16<BF16>(vf, pb[i / DBLK], acc_o[i % DBLK]);
                if constexpr (BF16) acc_o[i % DBLK] = mfma16<BF16>(vf, pl[i / DBLK], acc_o[i % DBLK]);
            });
        buf ^= 1;
        st = nxt;
    }
    lds_done_barrier();  // every wave is done with the stage buffers

    // ---- epilogue: lane holds O[slot j16][16*db + 4*g4 + e]
    bool write_final = a.splits == 1;
    bool gave_up = false;
    if constexpr (HAS_MASK) {
        if (side >= 0) {
            // one side of a cut row block: as in prefill_kernel, the first side to arrive
            // publishes its partial and raises the ready flag, the second waits for the
            // flag (bounded) and merges
            int *arrival = reinterpret_cast<int *>(m_lds + NW * MI * 64);
            const int64_t pu = ((int64_t)b * a.head_groups + hg) * (a.row_blocks >> 1) + pair;
            constexpr int PBYTES = DBLK * 64 * 16;  // one wave's partial
            write_final = pair_arrive(a, pu, arrival);
            if (!write_final) {
                const __amdgpu_buffer_rsrc_t mine = __builtin_amdgcn_make_buffer_rsrc(
                    a.pair_part + ((pu * 2 + side) * NW + wave) * (PBYTES / 4), 0, PBYTES, kRawBufferFlags);
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4v, acc_o[db]), mine,
                                                           (db * 64 + lane) * 16, 0, kAgentCoherent);
                if (g4 == 0) pair_store_ml(a, pu, side, slot, m_run, l_run);
                pair_ready(a, pu);
            } else {
                gave_up = pair_wait(a, pu, arrival);
            }
            if (write_final && !gave_up) {
                const int other = 1 - side;
                const float2 mlo = pair_load_ml(a, pu, other, slot);
                const float mo = mlo.x, lo = mlo.y;
                const float mx = fmaxf(m_run, mo);
                const float wa = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
                const float wb = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mx);
                const __amdgpu_buffer_rsrc_t theirs = __builtin_amdgcn_make_buffer_rsrc(
                    a.pair_part + ((pu * 2 + other) * NW + wave) * (PBYTES / 4), 0, PBYTES, kRawBufferFlags);
                // four blocks in flight at a time (one round trip each, not one per block)
#pragma unroll
                for (int d0 = 0; d0 < DBLK; d0 += 4) {
                    float4v x[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        x[jj] = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(
                                                                theirs, ((d0 + jj) * 64 + lane) * 16, 0, kAgentCoherent));
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) acc_o[d0 + jj] = acc_o[d0 + jj] * wa + x[jj] * wb;
                }
                l_run = wa * l_run + wb * lo;
            }
        }
    }
    if ((write_final || a.splits > 1) && row_ok) {
        const float sc = gave_up ? __builtin_nanf("") : write_final ? (l_run > 0.f ? 1.f / l_run : 0.f) : 1.f;
        if (!write_final && g4 == 0) {
            const int64_t unit = (((int64_t)split * a.batch + b) * a.n_heads + head) * a.rows + row;
            a.ml[unit] = make_float2(m_run, l_run);
        }
        float *dst = write_final ? a.o + b * a.o_bs + (int64_t)row * a.o_rs + (int64_t)head * a.o_hs
                                 : a.part + ((((int64_t)split * a.batch + b) * a.n_heads + head) * a.rows + row) * D;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) *reinterpret_cast<float4v *>(dst + 16 * db + 4 * g4) = acc_o[db] * sc;
    }
    __syncthreads();  // the next task reuses the LDS buffers
    }  // task
}

template <int D, bool BF16, int MASK>
hipError_t launch_narrow_dim(const PrefillArgs &a, const PrefillPlan *plan, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)plan->head_groups * plan->row_blocks * a.splits * a.batch));
    if constexpr (BF16) {
        if (!a.q_bf16) {
            hipLaunchKernelGGL((narrow_kernel<D, 8, true, MASK, true>), grid, dim3(512), 0, stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((narrow_kernel<D, 8, BF16, MASK, false>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_narrow_prefill(const PrefillArgs &a, const PrefillPlan *plan, bool bf16, hipStream_t stream) {
    const bool has_mask = a.mask != nullptr;
    const int mask = !has_mask ? 0 : a.mask_bf16 ? 2 : 1;
    auto by_type = [&](auto d_c) -> hipError_t {
        constexpr int D = decltype(d_c)::value;
        if (bf16) {
            return mask == 0 ? launch_narrow_dim<D, true, 0>(a, plan, stream)
                 : mask == 1 ? launch_narrow_dim<D, true, 1>(a, plan, stream)
                             : launch_narrow_dim<D, true, 2>(a, plan, stream);
        }
        return mask == 0 ? launch_narrow_dim<D, false, 0>(a, plan, stream)
             : mask == 1 ? launch_narrow_dim<D, false, 1>(a, plan, stream)
                         : launch_narrow_dim<D, false, 2>(a, plan, stream);
    };
    switch (plan->head_dim) {
    case 128: return by_type(std::integral_constant<int, 128>{});
    case 256: return by_type(std::integral_constant<int, 256>{});
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
