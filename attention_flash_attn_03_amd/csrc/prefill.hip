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
//  * K and V stages (64 or 32 rows) and the classified mask tiles stream into
//    LDS with global_load_lds_dwordx4 (no staging registers), XOR-swizzled so
//    both LDS read patterns are free of bank conflicts.  Stages are double
//    buffered: stage j+1 is requested right after the barrier that opens
//    stage j.  Q comes in and O goes out through LDS as whole rows
//    (coalesced), with the score scale folded into Q where that is exact
//    enough.
//  * exp2 with log2(e) folded into the score scale.  With f16 K/V, P is
//    rounded to f16 before P V and the running sum l is taken from the
//    rounded P, so the rounding cancels in O / l; with bf16 K/V, P enters P V
//    as a hi + lo pair of bf16 (two MFMAs).  O is rescaled only when some
//    lane's running max moved (lazy rescale).
//  * Masked calls pair row blocks p and RB-1-p across two workgroups that
//    split their unskipped stages evenly, whatever the mask shape; the side
//    that finishes a cut block second merges the two partial results
//    (agent-coherent buffer accesses and a relaxed atomic counter, no fence).
//    Calls with few query blocks split the KV range across workgroups with a
//    log-sum-exp combine pass.
#include "prefill_common.h"

namespace attn {
namespace {

// QSPLIT: f32 Q against bf16 K/V.  bf16 keeps 8 significant bits, which
// perturbs every score by about 2^-9 relative; Q is carried as hi + lo bf16
// parts (about 16 significant bits) and both products go into S.
//
// NW waves per workgroup; with head_dim 512 the waves pair up as two slices
// of 256 head-dim columns over the same 32 query slots (NS = 2) and add their
// partial scores through LDS; otherwise every wave has its own query slots.
// A stage is BK keys (64, or 32 at head_dim 512 so two stages fit in LDS);
// the tile codes cover 64 keys.
//
// Schedule of stage j (K/V of j are in buffer j%2, requested one stage ago):
//   touch mask(j) registers and wait for everything -> K(j), V(j), mask(j) landed
//   request mask(j+1) (registers) and K(j+1), V(j+1) (the other LDS buffer)
//   S^T = K Q^T, scale + mask, online softmax, O^T += V^T P^T
//   barrier (every wave is done with buffer j%2)
// so each stage's loads have a whole stage of compute to land, and no wait for
// a load the compiler can see ever drains the prefetch (loads retire in order,
// and the mask loads are always requested before the stage they belong to).
// MASK: 0 none, 1 f16, 2 bf16
template <int D, int NW, bool BF16, int MASK, bool QSPLIT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1))) void prefill_kernel(PrefillArgs a) {
    constexpr bool HAS_MASK = MASK != 0;
    constexpr bool MBF16 = MASK == 2;
    constexpr int NS = D > 256 ? 2 : 1;       // head-dim slices
    constexpr int DS = D / NS;                 // columns per wave
    constexpr int KSTEPS = DS / 16;            // MFMA k-steps of S over a slice
    constexpr int DBLK = DS / 32;              // 32-column O blocks per wave
    // keys per stage: two stages of K and V fit in LDS with room for the other resident
    // workgroups (512 * D bytes at 64 keys), and the f32-Q split at head_dim 256 stays
    // within the register file
    constexpr int BK = (D > 256 || (D == 256 && (NW == 2 || QSPLIT))) ? 32 : 64;
    constexpr int NB = BK / 32;                // 32-key blocks per stage
    constexpr int SPT = kTile / BK;            // stages per 64-key tile code
    constexpr int STAGE_ELEMS = BK * D;
    using KS = TileStream<D, NW, BK, kSwzK>;
    using VS = TileStream<D, NW, BK, kSwzV32>;
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2 * STAGE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2 * STAGE_ELEMS];
    __shared__ __attribute__((aligned(16))) float4v x_lds[NS > 1 ? NW * NB * 4 * 64 : 1];
    constexpr int QW = NW / NS;                // query waves
    constexpr int MI = 2 * NB;                 // mask DMA instructions per query wave per stage
    __shared__ __attribute__((aligned(1024))) uint4v m_lds[HAS_MASK ? 2 * QW * MI * 64 : 1];

    // A WT_ROWS x DS f32 tile per wave for staging rows of O out (and Q in), carved
    // from the K and V buffers (free before the first stage and after the last): half
    // the waves in each.
    constexpr int WT_PER = NW / 2 > 0 ? NW / 2 : 1;  // wave tiles per buffer
    constexpr int WT_ROWS = 32;
    constexpr int WT_BYTES = WT_ROWS * DS * 4;
    // Every launch shape stages its 32 rows in one pass.  (Staging in two passes of 16
    // rows gave wrong rows in the masked builds that used it, with a cause not found;
    // that shape is not built.)
    static_assert(WT_PER * WT_BYTES <= 2 * BK * D * 2, "staging tiles of 32 rows fit the K/V buffers");
    auto wave_tile = [&](int w) -> char * {
        return (w < WT_PER ? reinterpret_cast<char *>(k_lds) : reinterpret_cast<char *>(v_lds)) + (w % WT_PER) * WT_BYTES;
    };
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (!HAS_MASK) {
        // without a mask there is no classify pass and no pairing: only this write touches the status block
        if (blockIdx.x == 0 && threadIdx.x < kStatusWords) a.status[threadIdx.x] = 0u;
    }
    const int slice = wave % NS;
    const int qwave = wave / NS;
    const int half = lane >> 5;    // which 8-element k half of an MFMA operand this lane feeds
    const int col = lane & 31;     // query slot column inside the wave

    // 1-D grid: head group fastest (consecutive workgroups go to consecutive XCDs, so the
    // workgroups of one KV head share an L2), then row blocks, then split and batch.
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
    const int split_begin = split * a.tiles_per_split * SPT;
    const int split_end = min(split_begin + a.tiles_per_split * SPT, n_stages);

    // tile codes are read as dwords through the scalar cache (constant address space)
    auto code_row = [&](int rbx) -> const_u32 * {
        const int bh = a.blk_heads == 1 ? 0 : hg;
        return (const_u32 *)(a.blk + (((int64_t)b * a.blk_heads + bh) * a.row_blocks + rbx) * a.blk_stride);
    };
    // the tasks of this workgroup (row blocks and stage ranges; pairing of heavy and light
    // row blocks with a cut in the heavy one)
    const PrefillTasks tasks = prefill_tasks<SPT, HAS_MASK>(a, b, hg, idx, split_begin, split_end, n_stages, lane);
    const int rb0 = tasks.rb0, beg0 = tasks.beg0, end0 = tasks.end0, side0 = tasks.side0;
    const int rb1 = tasks.rb1, beg1 = tasks.beg1, end1 = tasks.end1, ntask = tasks.ntask, pair = tasks.pair;

    for (int task = 0; task < ntask; ++task) {
    const int rb = task == 0 ? rb0 : rb1;
    const int st_begin = task == 0 ? beg0 : beg1;
    const int st_end = task == 0 ? end0 : end1;
    const int side = task == 0 ? side0 : -1;

    // this lane's query slot
    const int slot = qwave * 32 + col;
    const int head = h0 + slot / a.rows_per_wg;
    const int row = rb * a.rows_per_wg + slot % a.rows_per_wg;
    const bool row_ok = row < a.rows;
    const int row_c = row_ok ? row : a.rows - 1;

    // ---- Q fragment: B operand of S^T = K Q^T, k = slice*DS + 16*ks + 8*half + i.
    // f32 Q over the whole head dim goes straight into registers in fragment order (below,
    // with the first K/V stage); otherwise the wave's query rows (its DS columns) are read
    // with one contiguous row segment per load instruction into its LDS tile, then picked
    // up in fragment order.
    // Q is rounded to the K/V type anyway (f16, or a bf16 hi + lo pair), so the score
    // scale and log2(e) are folded in before rounding; only bf16 Q against bf16 K/V is
    // used as given (re-rounding would add error) and its scores are scaled after the
    // MFMA.  With two head-dim slices the scaling stays after the MFMA (measured faster:
    // it rides along with the exchange of the slices' partial scores).
    constexpr bool PRESCALE = (!BF16 || QSPLIT) && NS == 1;
    const float q_scale = PRESCALE ? a.score_scale : 1.f;
    const float post_scale = PRESCALE ? 1.f : a.score_scale;
    uint4v qf[KSTEPS];
    uint4v qlo[QSPLIT ? KSTEPS : 1];

    const uint16_t *mrow = nullptr;
    if constexpr (HAS_MASK) {
        mrow = (const uint16_t *)a.mask + b * a.m_bs + head * a.m_hs + (int64_t)row_c * a.m_rs;
    }

    float16v acc_o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_run = -INFINITY;  // reference max of the log2-scaled scores (at most kRescaleThreshold stale)
    float l_run = 0.f;        // running sum of the rounded probabilities

    const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_bs + kvh * a.k_hs;
    const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_bs + kvh * a.v_hs;
    const_u32 *blk_row = nullptr;
    if constexpr (HAS_MASK) blk_row = code_row(rb);
    auto stage_code = [&](int st) -> int {
        if constexpr (HAS_MASK) {
            const int t = st / SPT;
            return (int)((blk_row[t >> 2] >> (8 * (t & 3))) & 0xffu);
        } else {
            return TILE_OPEN;
        }
    };
    auto next_stage = [&](int from) {
        int st = from;
        while (st < st_end && stage_code(st) == TILE_SKIP) ++st;
        return st < st_end ? st : st_end;
    };
    // Mask of a stage.  Full stages of a 16-byte aligned mask are streamed into LDS
    // beside K and V: instruction i of a query wave fetches, for each of its 32 query
    // rows, the 8-key chunks 2i (lanes 0..31) and 2i+1 (lanes 32..63), so that all 64
    // lanes reading one chunk touch 512 contiguous bytes.  Other stages (the ragged
    // last one, or a mask of other alignment) are read from memory where they are used.
    auto mask_in_lds = [&](int st) { return a.mask_dma && st * BK + BK <= a.kv_len; };
    auto issue_mask = [&](int st, int bufi) {
        const uint32_t mbase = (uint32_t)(uintptr_t)(lds_void *)(m_lds + (bufi * QW + qwave) * MI * 64);
        const uint16_t *src = mrow + st * BK + 8 * half;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(mbase + i * 1024);
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src + 16 * i) : "memory");
        }
    };
    // raw mask values of this lane's keys in stage st: key0 + 32*bb + 8*q4 + 4*half + e
    auto load_mask = [&](uint2 (&mr)[NB][4], int st, int bufi) {
        const int key0 = st * BK;
        if (mask_in_lds(st)) {
            const uint4v *mb = m_lds + (bufi * QW + qwave) * MI * 64;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int c = 4 * bb + q4;
                    mr[bb][q4] = *reinterpret_cast<const uint2 *>(
                        reinterpret_cast<const char *>(mb + (c >> 1) * 64 + (c & 1) * 32 + col) + 8 * half);
                }
        } else {
            // any alignment, any tail: element loads from clamped (in-bounds) keys
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int kf = key0 + 32 * bb + 8 * q4 + 4 * half;
                    uint16_t m16[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) m16[e] = mrow[min(kf + e, a.kv_len - 1)];
                    mr[bb][q4] = make_uint2(pack2(m16[0], m16[1]), pack2(m16[2], m16[3]));
                }
        }
    };

    KS kstream;
    VS vstream;
    kstream.init(lane, wave, a.k_rs);
    vstream.init(lane, wave, a.v_rs);

    // LDS byte offsets of the MFMA operand reads.  The swizzles permute only the low
    // bits of a chunk index, so every read is one of a few lane offsets plus a
    // compile-time immediate (the ds_read offset field), and no per-step address
    // has to be held in a register.
    //  K (A operand of S^T): k-step ks of key block bb reads row 32*bb + col, logical
    //    chunk slice*DS/8 + 2*ks + half, stored at chunk ^ (col & 15).  For ks = 8*g + r
    //    that is chunk 16*g + ((2r + half) ^ (col & 15)) past the slice: k_off[r] + g*256
    //    + bb*32*D*2.
    uint32_t k_off[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        k_off[r] = (uint32_t)((col * D + slice * DS + 8 * ((2 * r + half) ^ (col & 15))) * 2);
    //  V (transposing reads for the A operand of O^T): lane j of 16-lane group g reads row
    //    16*u + vr (and vr + 8) with vr = 4*(g/2) + j/4, logical chunk slice*DS/8 + 4*db + l0
    //    with l0 = 2*(g&1) + (j&3)/2, element 4*(j&1); the chunk is stored at chunk ^ 4*(vr&3),
    //    i.e. 4*(db ^ (vr&3)) + l0 with only db's low two bits changed: v_off[db&3] +
    //    64*(db & ~3) + u*32*D (+ 16*D for the rows vr + 8).
    uint32_t v_off[4];
    {
        const int g16 = lane >> 4, j16 = lane & 15;
        const int vr = 4 * (g16 >> 1) + (j16 >> 2);
        const int l0 = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v_off[q] = (uint32_t)((vr * D + 4 * (j16 & 1) + 8 * (slice * (DS / 8) + 4 * (q ^ (vr & 3)) + l0)) * 2);
    }

    int st = next_stage(st_begin);
    int buf = 0;
    auto issue_first_stage = [&]() {
        if (st < st_end) {
            if (HAS_MASK && slice == 0 && stage_code(st) == TILE_MASKED && mask_in_lds(st)) issue_mask(st, 0);
            const bool full = st * BK + BK <= a.kv_len;
            kstream.issue(k_lds, kbase, a.k_rs, st * BK, a.kv_len, wave, full);
            vstream.issue(v_lds, vbase, a.v_rs, st * BK, a.kv_len, wave, full);
        }
    };
    if (NS == 1 && D <= 256 && !a.q_bf16) {
        // f32 Q over the whole head dim: each lane reads its query row's fragment straight into
        // registers, and the first K/V stage is requested before those rows are converted, so
        // the two share one memory round trip
        const float *qrow = reinterpret_cast<const float *>(a.q) + b * a.q_bs + (int64_t)row_c * a.q_rs +
                            (int64_t)head * a.q_hs + 8 * half;
        float4v qraw[KSTEPS][2];
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            qraw[ks][0] = *reinterpret_cast<const float4v *>(qrow + 16 * ks);
            qraw[ks][1] = *reinterpret_cast<const float4v *>(qrow + 16 * ks + 4);
        }
        issue_first_stage();
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
        {
            char *tile = wave_tile(wave);
            // rows of the pass go straight into the tile with LDS DMA: instruction `it` fills
            // 64 consecutive 16-byte slots (QRPI rows); the lane that fills slot j of row tr
            // fetches chunk j ^ (tr & 15) of that row, so chunk c lands at slot c ^ (tr & 15)
            auto stage_rows = [&](auto esz_c, int pass) __attribute__((always_inline)) {
                constexpr int ESZ = decltype(esz_c)::value;
                constexpr int QCPR = DS * ESZ / 16;       // 16-byte chunks per row
                const uint32_t tbase = (uint32_t)(uintptr_t)(lds_void *)tile;
    #pragma unroll 1
                for (int it = 0; it < WT_ROWS * QCPR / 64; ++it) {
                    // instruction `it` fills 16-byte slots it*64 .. it*64+63 of the tile
                    const int slot_i = it * 64 + lane;
                    const int tr = slot_i / QCPR;
                    const int c = (slot_i % QCPR) ^ (tr & 15);
                    const int sl = qwave * 32 + pass * WT_ROWS + tr;
                    const int rh = h0 + sl / a.rows_per_wg;
                    int rr = rb * a.rows_per_wg + sl % a.rows_per_wg;
                    rr = rr < a.rows ? rr : a.rows - 1;
                    const char *src = reinterpret_cast<const char *>(a.q) +
                                      (b * a.q_bs + (int64_t)rr * a.q_rs + rh * a.q_hs + slice * DS) * ESZ + c * 16;
                    const uint32_t m0 = __builtin_amdgcn_readfirstlane(tbase + it * 1024);
                    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory");
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            };
            const int tr = col % WT_ROWS;
            // tile rows hold logical chunk c at c ^ (tr & 15): as for the K reads, the chunks a lane
            // picks up are a few lane offsets plus immediates.  bf16 rows: chunk 2*ks + half;
            // f32 rows: chunks 4*ks + 2*half + e (e = 0, 1).
            uint32_t qo[8];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                qo[r] = a.q_bf16 ? (uint32_t)(tr * (DS * 2) + (((2 * r + half) ^ (tr & 15)) * 16))
                                 : (uint32_t)(tr * (DS * 4) + (((4 * (r >> 1) + 2 * half + (r & 1)) ^ (tr & 15)) * 16));
#pragma unroll
            for (int pass = 0; pass < 32 / WT_ROWS; ++pass) {
                if (a.q_bf16) {
                    stage_rows(std::integral_constant<int, 2>{}, pass);
                    if (col / WT_ROWS == pass) {
#pragma unroll
                        for (int ks = 0; ks < KSTEPS; ++ks) {
                            const uint4v raw = *reinterpret_cast<const uint4v *>(tile + qo[ks & 7] + (ks >> 3) * 256);
                            if constexpr (BF16) {
                                qf[ks] = raw;
                            } else {
                                uint4v cv;
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const float lo = bf16_bits_to_f32((uint16_t)(raw[e] & 0xffffu)) * q_scale;
                                    const float hi = bf16_bits_to_f32((uint16_t)(raw[e] >> 16)) * q_scale;
                                    cv[e] = pack2(to_kv16<false>(lo), to_kv16<false>(hi));
                                }
                                qf[ks] = cv;
                            }
                        }
                    }
                } else {
                    stage_rows(std::integral_constant<int, 4>{}, pass);
                    if (col / WT_ROWS == pass) {
#pragma unroll
                        for (int ks = 0; ks < KSTEPS; ++ks) {
                            const char *row = tile + (ks >> 2) * 256;
                            const float4v x0 = *reinterpret_cast<const float4v *>(row + qo[2 * (ks & 3)]) * q_scale;
                            const float4v x1 = *reinterpret_cast<const float4v *>(row + qo[2 * (ks & 3) + 1]) * q_scale;
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
                }
            }
            if (!row_ok) {
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) {
                    qf[ks] = uint4v{0u, 0u, 0u, 0u};
                    if constexpr (QSPLIT) qlo[ks] = qf[ks];
                }
            }
            __syncthreads();  // every wave has its Q before the first K/V stage overwrites the tiles
        }
        issue_first_stage();
    }
    while (st < st_end) {
        const int code = stage_code(st);
        const int nxt = next_stage(st + 1);
        const int key0 = st * BK;
        const bool full_stage = key0 + BK <= a.kv_len;
        const bool use_mask = HAS_MASK && code == TILE_MASKED && slice == 0;

        wait_all_barrier();  // K, V and mask of this stage landed (all requested one stage ago)

        // Request stage nxt into the other buffers.  Issued together the loads stall the wave
        // until the memory pipeline has taken them; a full stage is therefore issued one
        // instruction at a time between the S MFMAs below (a ragged or widely strided stage
        // at once, here).
        const bool nfull = nxt < st_end && nxt * BK + BK <= a.kv_len && a.k_rs < kOff32Stride &&
                           a.v_rs < kOff32Stride;
        if (nxt < st_end && !nfull) {
            if (HAS_MASK && slice == 0 && stage_code(nxt) == TILE_MASKED && mask_in_lds(nxt)) issue_mask(nxt, buf ^ 1);
            kstream.issue(k_lds + (buf ^ 1) * STAGE_ELEMS, kbase, a.k_rs, nxt * BK, a.kv_len, wave, false);
            vstream.issue(v_lds + (buf ^ 1) * STAGE_ELEMS, vbase, a.v_rs, nxt * BK, a.kv_len, wave, false);
        }
        const bool nmask = HAS_MASK && nfull && slice == 0 && stage_code(nxt) == TILE_MASKED && mask_in_lds(nxt);
        const char *kst = KS::stage_ptr(kbase, a.k_rs, nxt * BK, wave);
        const char *vst = VS::stage_ptr(vbase, a.v_rs, nxt * BK, wave);
        uint16_t *kdst = k_lds + (buf ^ 1) * STAGE_ELEMS;
        uint16_t *vdst = v_lds + (buf ^ 1) * STAGE_ELEMS;
        const uint32_t mdst = (uint32_t)(uintptr_t)(lds_void *)(m_lds + ((buf ^ 1) * QW + qwave) * MI * 64);
        // instruction n of the next stage: mask chunks first, then K and V alternately
        constexpr int NDMA = (HAS_MASK ? MI : 0) + 2 * KS::NLD;
        static_assert(KS::NLD == VS::NLD, "K and V stream alike");
        auto dma_one = [&](auto n_c) __attribute__((always_inline)) {
            constexpr int n = decltype(n_c)::value;
            if constexpr (HAS_MASK && n < MI) {
                if (nmask) {
                    const uint32_t m0 = __builtin_amdgcn_readfirstlane(mdst + n * 1024);
                    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0),
                                 "v"(mrow + nxt * BK + 8 * half + 16 * n)
                                 : "memory");
                }
            } else {
                constexpr int j = n - (HAS_MASK ? MI : 0);
                if constexpr (j % 2 == 0) kstream.issue_one(kdst, kst, a.k_rs, j / 2, wave);
                else vstream.issue_one(vdst, vst, a.v_rs, j / 2, wave);
            }
        };
        const uint16_t *kt_lds = k_lds + buf * STAGE_ELEMS;
        const uint16_t *vt_lds = v_lds + buf * STAGE_ELEMS;

        // ---- S^T (BK keys x 32 queries) over this wave's head-dim slice
        float16v s[NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[bb][r] = 0.f;
        // step i: k-step i / NB of key block i % NB
        lds_pipeline<NB * KSTEPS, kLdsAhead, uint4v>(
            [&](int i) __attribute__((always_inline)) {
                const int bb = i % NB, ks = i / NB;
                return *reinterpret_cast<const uint4v *>(reinterpret_cast<const char *>(kt_lds) + k_off[ks & 7] +
                                                         (ks >> 3) * 256 + bb * 32 * D * 2);
            },
            [&](int i, const uint4v &kf) __attribute__((always_inline)) {
                s[i % NB] = mfma32<BF16>(kf, qf[i / NB], s[i % NB]);
                if constexpr (QSPLIT) s[i % NB] = mfma32<BF16>(kf, qlo[i / NB], s[i % NB]);
                if (nfull) {
                    // instruction n at step n * (S steps) / NDMA
                    static_for<NDMA>([&](auto n_c) __attribute__((always_inline)) {
                        if (i == (decltype(n_c)::value * NB * KSTEPS) / NDMA) dma_one(n_c);
                    });
                }
            });

        // ---- scale and mask (log2 units); this lane holds keys key0 + 32*bb + 8*(r/4) + 4*half + r%4
        if (use_mask) {
            uint2 mcur[NB][4];
            load_mask(mcur, st, buf);
            auto add_mask = [&](auto bf_c) __attribute__((always_inline)) {
                constexpr bool MBF = decltype(bf_c)::value;
#pragma unroll
                for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t word = e < 2 ? mcur[bb][q4].x : mcur[bb][q4].y;
                            const uint16_t m16 = (uint16_t)(word >> (16 * (e & 1)));
                            const float mv = MBF ? bf16_bits_to_f32(m16) : f16_bits_to_f32(m16);
                            const float x = s[bb][4 * q4 + e];
                            s[bb][4 * q4 + e] = PRESCALE ? fmaf(mv, kLog2e, x) : fmaf(x, post_scale, mv * kLog2e);
                        }
            };
            add_mask(std::integral_constant<bool, MBF16>{});
        } else if constexpr (!PRESCALE) {
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[bb][r] *= post_scale;
        }
        if constexpr (NS > 1) {
            // add the other slice's partial scores
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4)
                    x_lds[((wave * NB + bb) * 4 + r4) * 64 + lane] =
                        float4v{s[bb][4 * r4], s[bb][4 * r4 + 1], s[bb][4 * r4 + 2], s[bb][4 * r4 + 3]};
            lds_done_barrier();
            const int other = qwave * NS + (1 - slice);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const float4v x = x_lds[((other * NB + bb) * 4 + r4) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[bb][4 * r4 + e] += x[e];
                }
        }
        if (!full_stage) {
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (key0 + 32 * bb + 8 * (r >> 2) + 4 * half + (r & 3) >= a.kv_len) s[bb][r] = -INFINITY;
        }

        // ---- online softmax for this lane's query (BK/2 keys here, BK/2 in lane ^ 32)
        float mx = -INFINITY;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[bb][r]);
        mx = max_with_other_half(mx);
        const bool grow = mx > m_run + kRescaleThreshold;  // also true for the first visible key
        const float m_new = grow ? mx : m_run;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        float rowsum = 0.f;
        uint4v pb[2 * NB];  // B operands of O^T += V^T P^T: pb[2*bb + e] holds regs 8e..8e+7 of s[bb]
        uint4v pl[BF16 ? 2 * NB : 1];  // bf16: the low parts of P
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint32_t w[4], wl[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p0 = __builtin_amdgcn_exp2f(s[bb][8 * e + 2 * i] - m_use);
                    const float p1 = __builtin_amdgcn_exp2f(s[bb][8 * e + 2 * i + 1] - m_use);
                    if constexpr (BF16) pack_p_bf16(p0, p1, w[i], wl[i], rowsum);
                    else w[i] = pack_p_f16(p0, p1, rowsum);
                }
                pb[2 * bb + e] = uint4v{w[0], w[1], w[2], w[3]};
                if constexpr (BF16) pl[2 * bb + e] = uint4v{wl[0], wl[1], wl[2], wl[3]};
            }
        rowsum = sum_with_other_half(rowsum);
        l_run = l_run * alpha + rowsum;
        m_run = m_new;
        if (__ballot(grow)) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_o[db][r] = scale_acc(acc_o[db][r], alpha);
        }

        // ---- O^T[d][query] += V^T[d][key] P^T[key][query]
        // A operand slot i of lane (m, half) is key 32*bb + 16*e + 8*(i/4) + 4*half + i%4, column m.
        // A 16-lane group g reads 4 keys x 16 columns per ds_read_b64_tr_b16: lane j of the
        // group points at row kb + j/4, columns c0 + 4*(j%4) .. +3; lane j receives
        // rows kb..kb+3 of column c0 + j.
        // step i: P^T slice u = i / DBLK (key block u / 2, half u % 2) into O block i % DBLK
        lds_pipeline<2 * NB * DBLK, kLdsAhead, uint4v>(
            [&](int i) __attribute__((always_inline)) {
                const int u = i / DBLK, db = i % DBLK;  // rows 16u + vr (slots 0..3) and 16u + vr + 8 (slots 4..7)
                const char *p0 = reinterpret_cast<const char *>(vt_lds) + v_off[db & 3] + 64 * (db & ~3) + u * 32 * D;
                return read_tr16_pair(reinterpret_cast<const uint16_t *>(p0),
                                      reinterpret_cast<const uint16_t *>(p0 + 16 * D));
            },
            [&](int i, const uint4v &vf) __attribute__((always_inline)) {
                acc_o[i % DBLK] = mfma32<BF16>(vf, pb[i / DBLK], acc_o[i % DBLK]);
                if constexpr (BF16) acc_o[i % DBLK] = mfma32<BF16>(vf, pl[i / DBLK], acc_o[i % DBLK]);
            });
        buf ^= 1;
        st = nxt;
    }
    lds_done_barrier();  // every wave is done with the stage buffers, which the epilogue reuses

    // ---- epilogue: this lane holds O^T columns query `col`, rows d = slice*DS + 32*db + 8*(r/4) + 4*half + r%4.
    // Split and pair partials are kept in this fragment order (each store instruction
    // writes 1 KB contiguous); rows of O and of the split partials go out through an
    // LDS tile of the wave (the K/V buffers are free now), one contiguous row segment
    // per store instruction.
    bool write_final = a.splits == 1;
    bool gave_up = false;
    if constexpr (HAS_MASK) {
        if (side >= 0) {
            // one side of a cut row block.  The side that arrives first publishes its partial
            // and raises the pair's ready flag; the side that arrives second waits for that
            // flag (the first side has arrived by then and owes only its stores, so the wait
            // ends) and merges both into the output.
            // the protocol's LDS word is the second mask buffer: the next task writes it only
            // after the barrier that starts its first stage
            int *arrival = reinterpret_cast<int *>(m_lds + QW * MI * 64);
            const int64_t pu = ((int64_t)b * a.head_groups + hg) * (a.row_blocks >> 1) + pair;
            constexpr int PBYTES = DBLK * 4 * 64 * 16;  // one wave's partial
            write_final = pair_arrive(a, pu, arrival);
            if (!write_final) {
                const __amdgpu_buffer_rsrc_t mine = __builtin_amdgcn_make_buffer_rsrc(
                    a.pair_part + ((pu * 2 + side) * NW + wave) * (PBYTES / 4), 0, PBYTES, kRawBufferFlags);
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(uint4v, float4v{acc_o[db][4 * r4], acc_o[db][4 * r4 + 1],
                                                               acc_o[db][4 * r4 + 2], acc_o[db][4 * r4 + 3]}),
                            mine, ((db * 4 + r4) * 64 + lane) * 16, 0, kAgentCoherent);
                if (slice == 0 && half == 0) pair_store_ml(a, pu, side, slot, m_run, l_run);
                pair_ready(a, pu);
            } else {
                gave_up = pair_wait(a, pu, arrival);
            }
            if (write_final && !gave_up) {
                // the other side's partial was complete before its ready flag, which this
                // side has observed
                const int other = 1 - side;
                const float2 mlo = pair_load_ml(a, pu, other, slot);
                const float mo = mlo.x, lo = mlo.y;
                const float mx = fmaxf(m_run, mo);
                const float wa = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
                const float wb = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mx);
                const __amdgpu_buffer_rsrc_t theirs = __builtin_amdgcn_make_buffer_rsrc(
                    a.pair_part + ((pu * 2 + other) * NW + wave) * (PBYTES / 4), 0, PBYTES, kRawBufferFlags);
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const float4v x = __builtin_bit_cast(
                            float4v, __builtin_amdgcn_raw_buffer_load_b128(theirs, ((db * 4 + r4) * 64 + lane) * 16, 0,
                                                                           kAgentCoherent));
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc_o[db][4 * r4 + e] = acc_o[db][4 * r4 + e] * wa + x[e] * wb;
                    }
                l_run = wa * l_run + wb * lo;
            }
        }
    }
    if (write_final || a.splits > 1) {
        // rows of this wave's 32 x DS tile: final O (normalised), or a split partial
        const float sc = gave_up ? __builtin_nanf("") : write_final ? (l_run > 0.f ? 1.f / l_run : 0.f) : 1.f;
        char *tile = wave_tile(wave);
        if (!write_final && slice == 0 && half == 0 && row_ok) {
            const int64_t unit = (((int64_t)split * a.batch + b) * a.n_heads + head) * a.rows + row;
            a.ml[unit] = make_float2(m_run, l_run);
        }
        constexpr int CPR = DS / 4;      // 16-byte chunks per row
        // this lane's chunks of its row: 8*db + 2*r4 + half, stored at chunk ^ (tr & 15), i.e.
        // eo[2*(db&1) ... ] lane offsets plus 256*(db >> 1)
        const int etr = col % WT_ROWS;
        uint32_t eo[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
            eo[r] = (uint32_t)(etr * (DS * 4) + (((8 * (r >> 2) + 2 * (r & 3) + half) ^ (etr & 15)) * 16));
#pragma unroll
        for (int pass = 0; pass < 32 / WT_ROWS; ++pass) {
            if (col / WT_ROWS == pass) {
#pragma unroll
                for (int db = 0; db < DBLK; ++db)
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        float4v x;
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] = acc_o[db][4 * r4 + e] * sc;
                        *reinterpret_cast<float4v *>(tile + eo[4 * (db & 1) + r4] + (db >> 1) * 256) = x;
                    }
            }
#pragma unroll
            for (int it = 0; it < WT_ROWS * CPR / 64; ++it) {
                // store instruction `it` writes 16-byte chunks it*64 .. it*64+63 of the tile's rows
                const int tr = (it * 64 + lane) / CPR;
                const int c = (it * 64 + lane) % CPR;
                const int sl = qwave * 32 + pass * WT_ROWS + tr;
                const int rh = h0 + sl / a.rows_per_wg;
                const int rr = rb * a.rows_per_wg + sl % a.rows_per_wg;
                const float4v x = *reinterpret_cast<const float4v *>(tile + tr * (DS * 4) + ((c ^ (tr & 15)) * 16));
                if (rr < a.rows) {
                    float *dst = write_final
                                     ? a.o + b * a.o_bs + (int64_t)rr * a.o_rs + rh * a.o_hs
                                     : a.part + ((((int64_t)split * a.batch + b) * a.n_heads + rh) * a.rows + rr) * D;
                    *reinterpret_cast<float4v *>(dst + slice * DS + 4 * c) = x;
                }
            }
        }
    }
    __syncthreads();  // the next task reuses the LDS tiles
    }  // task
}

// wide_kernel: head_dim 512 with every wave over the whole head dimension.  Four
// waves of 32 query slots make a 128-slot workgroup: each K/V byte feeds twice the
// queries of the two-slice layout and no partial scores are exchanged between
// waves.  Q (f16, or bf16 against bf16 K/V) lives in 128 VGPRs and O^T in all 256
// AGPRs, so the kernel keeps no other per-lane array: MFMA operand and mask reads
// are lane offsets plus immediates, Q is converted eight k-steps at a time, and O
// leaves straight from the accumulators.  No KV split and no row-block pairing:
// workgroup i takes the i-th (head group, row block, batch) item with the last row
// blocks (the heaviest under a causal frontier) dispatched first, so the hardware's
// in-order dispatch balances the tail.
template <int D, bool BF16, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void wide_kernel(PrefillArgs a) {
    constexpr int NW = 4;
    constexpr bool HAS_MASK = MASK != 0;
    constexpr bool MBF16 = MASK == 2;
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int BK = 32;                     // keys per stage: two stages of K and V are 128 KB
    constexpr int NB = BK / 32;
    constexpr int SPT = kTile / BK;
    constexpr int STAGE_ELEMS = BK * D;
    constexpr int MI = 2 * NB;                 // mask DMA instructions per wave per stage
    using KS = TileStream<D, NW, BK, kSwzK>;
    using VS = TileStream<D, NW, BK, kSwzV32>;
    __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2 * STAGE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2 * STAGE_ELEMS];
    __shared__ __attribute__((aligned(1024))) uint4v m_lds[HAS_MASK ? 2 * NW * MI * 64 : 1];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5;
    const int col = lane & 31;
    if constexpr (!HAS_MASK) {
        if (blockIdx.x == 0 && threadIdx.x < kStatusWords) a.status[threadIdx.x] = 0u;
    }
    int lin = blockIdx.x;
    const int hg = lin % a.head_groups;
    lin /= a.head_groups;
    const int rb = a.row_blocks - 1 - lin % a.row_blocks;
    const int b = lin / a.row_blocks;
    const int h0 = hg * a.heads_per_wg;
    const int kvh = h0 / a.group;
    const int n_stages = (a.kv_len + BK - 1) / BK;

    const int slot = wave * 32 + col;
    const int head = h0 + slot / a.rows_per_wg;
    const int row = rb * a.rows_per_wg + slot % a.rows_per_wg;
    const bool row_ok = row < a.rows;
    const int row_c = row_ok ? row : a.rows - 1;

    const_u32 *blk_row = nullptr;
    if constexpr (HAS_MASK)
        blk_row = (const_u32 *)(a.blk + (((int64_t)b * a.blk_heads + (a.blk_heads == 1 ? 0 : hg)) * a.row_blocks + rb) *
                                            a.blk_stride);
    auto stage_code = [&](int st) -> int {
        if constexpr (HAS_MASK) {
            const int t = st / SPT;
            return (int)((blk_row[t >> 2] >> (8 * (t & 3))) & 0xffu);
        } else {
            return TILE_OPEN;
        }
    };
    auto next_stage = [&](int from) {
        int st = from;
        while (st < n_stages && stage_code(st) == TILE_SKIP) ++st;
        return st;
    };
    const uint16_t *mrow = nullptr;
    if constexpr (HAS_MASK) mrow = (const uint16_t *)a.mask + b * a.m_bs + head * a.m_hs + (int64_t)row_c * a.m_rs;
    auto mask_in_lds = [&](int st) { return a.mask_dma && st * BK + BK <= a.kv_len; };
    // mask of a stage into this wave's LDS region: instruction i fetches, for each of the
    // wave's 32 query rows, the 8-key chunks 2i (lanes 0..31) and 2i+1 (lanes 32..63)
    auto issue_mask = [&](int st, int bufi) {
        const uint32_t mbase = (uint32_t)(uintptr_t)(lds_void *)(m_lds + (bufi * NW + wave) * MI * 64);
        const uint16_t *src = mrow + st * BK + 8 * half;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const uint32_t m0 = __builtin_amdgcn_readfirstlane(mbase + i * 1024);
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src + 16 * i) : "memory");
        }
    };

    const uint16_t *kbase = (const uint16_t *)a.k + b * a.k_bs + kvh * a.k_hs;
    const uint16_t *vbase = (const uint16_t *)a.v + b * a.v_bs + kvh * a.v_hs;
    KS kstream;
    VS vstream;
    kstream.init(lane, wave, a.k_rs);
    vstream.init(lane, wave, a.v_rs);
    int st = next_stage(0);
    auto issue_stage = [&](int s_, int bufi) {
        if (HAS_MASK && stage_code(s_) == TILE_MASKED && mask_in_lds(s_)) issue_mask(s_, bufi);
        const bool full = s_ * BK + BK <= a.kv_len;
        kstream.issue(k_lds + bufi * STAGE_ELEMS, kbase, a.k_rs, s_ * BK, a.kv_len, wave, full);
        vstream.issue(v_lds + bufi * STAGE_ELEMS, vbase, a.v_rs, s_ * BK, a.kv_len, wave, full);
    };

    // ---- Q fragments: B operand of S^T = K Q^T, k = 16*ks + 8*half + i.  f16 K/V: scale*log2(e)
    // folded in before rounding; bf16 Q against bf16 K/V is used as given and S is scaled after.
    constexpr bool PRESCALE = !BF16;
    uint4v qf[KSTEPS];
    if (!a.q_bf16) {
        const float *qrow = reinterpret_cast<const float *>(a.q) + b * a.q_bs + (int64_t)row_c * a.q_rs +
                            (int64_t)head * a.q_hs + 8 * half;
#pragma unroll
        for (int c0 = 0; c0 < KSTEPS; c0 += 8) {
            float4v raw[8][2];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                raw[j][0] = *reinterpret_cast<const float4v *>(qrow + 16 * (c0 + j));
                raw[j][1] = *reinterpret_cast<const float4v *>(qrow + 16 * (c0 + j) + 4);
            }
            if (c0 == 0 && st < n_stages) issue_stage(st, 0);  // the first stage shares the round trip
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4v x0 = raw[j][0] * a.score_scale, x1 = raw[j][1] * a.score_scale;
                uint4v cv;
                cv[0] = pack2(to_kv16<BF16>(x0[0]), to_kv16<BF16>(x0[1]));
                cv[1] = pack2(to_kv16<BF16>(x0[2]), to_kv16<BF16>(x0[3]));
                cv[2] = pack2(to_kv16<BF16>(x1[0]), to_kv16<BF16>(x1[1]));
                cv[3] = pack2(to_kv16<BF16>(x1[2]), to_kv16<BF16>(x1[3]));
                qf[c0 + j] = row_ok ? cv : uint4v{0u, 0u, 0u, 0u};
            }
        }
    } else {
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(a.q) + b * a.q_bs + (int64_t)row_c * a.q_rs +
                               (int64_t)head * a.q_hs + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const uint4v *>(qrow + 16 * ks);
        if (st < n_stages) issue_stage(st, 0);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            if constexpr (!BF16) {
                uint4v cv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf16_bits_to_f32((uint16_t)(qf[ks][e] & 0xffffu)) * a.score_scale;
                    const float hi = bf16_bits_to_f32((uint16_t)(qf[ks][e] >> 16)) * a.score_scale;
                    cv[e] = pack2(to_kv16<false>(lo), to_kv16<false>(hi));
                }
                qf[ks] = cv;
            }
            if (!row_ok) qf[ks] = uint4v{0u, 0u, 0u, 0u};
        }
    }
    const float post_scale = PRESCALE ? 1.f : a.score_scale;

    // MFMA operand reads as lane offsets plus immediates (layouts as in prefill_kernel)
    uint32_t k_off[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) k_off[r] = (uint32_t)((col * D + 8 * ((2 * r + half) ^ (col & 15))) * 2);
    uint32_t v_off[4];
    {
        const int g16 = lane >> 4, j16 = lane & 15;
        const int vr = 4 * (g16 >> 1) + (j16 >> 2);
        const int l0 = 2 * (g16 & 1) + ((j16 & 3) >> 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) v_off[q] = (uint32_t)((vr * D + 4 * (j16 & 1) + 8 * (4 * (q ^ (vr & 3)) + l0)) * 2);
    }

    float16v acc_o[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[db][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    int buf = 0;
    while (st < n_stages) {
        const int code = stage_code(st);
        const int nxt = next_stage(st + 1);
        const int key0 = st * BK;
        const bool full_stage = key0 + BK <= a.kv_len;
        wait_all_barrier();  // this stage's K, V and mask landed (requested one stage ago)
        // The next stage's loads.  Issued together they stall the wave until the memory
        // pipeline has taken them (72 KB per stage per CU); a full stage is therefore
        // issued one instruction at a time between the S MFMAs below.  A ragged or widely
        // strided stage is issued at once here.
        const bool nfull = nxt < n_stages && nxt * BK + BK <= a.kv_len && a.k_rs < kOff32Stride &&
                           a.v_rs < kOff32Stride;
        if (nxt < n_stages && !nfull) issue_stage(nxt, buf ^ 1);
        const bool nmask = HAS_MASK && nfull && stage_code(nxt) == TILE_MASKED && mask_in_lds(nxt);
        const char *kst = KS::stage_ptr(kbase, a.k_rs, nxt * BK, wave);
        const char *vst = VS::stage_ptr(vbase, a.v_rs, nxt * BK, wave);
        uint16_t *kdst = k_lds + (buf ^ 1) * STAGE_ELEMS;
        uint16_t *vdst = v_lds + (buf ^ 1) * STAGE_ELEMS;
        const uint32_t mdst = (uint32_t)(uintptr_t)(lds_void *)(m_lds + ((buf ^ 1) * NW + wave) * MI * 64);
        // instruction n of the next stage: mask chunks first, then K and V alternately
        constexpr int NDMA = (HAS_MASK ? MI : 0) + 2 * KS::NLD;
        auto dma_one = [&](auto n_c) __attribute__((always_inline)) {
            constexpr int n = decltype(n_c)::value;
            if constexpr (HAS_MASK && n < MI) {
                if (nmask) {
                    const uint32_t m0 = __builtin_amdgcn_readfirstlane(mdst + n * 1024);
                    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0),
                                 "v"(mrow + nxt * BK + 8 * half + 16 * n)
                                 : "memory");
                }
            } else {
                constexpr int j = n - (HAS_MASK ? MI : 0);
                if constexpr (j % 2 == 0) kstream.issue_one(kdst, kst, a.k_rs, j / 2, wave);
                else vstream.issue_one(vdst, vst, a.v_rs, j / 2, wave);
            }
        };
        const char *kt = reinterpret_cast<const char *>(k_lds + buf * STAGE_ELEMS);
        const char *vt = reinterpret_cast<const char *>(v_lds + buf * STAGE_ELEMS);

        float16v s;
        // mask values of this stage from LDS, requested eight MFMAs before the end of S so
        // that their latency hides under the matrix work
        const bool mask_lds_now = HAS_MASK && code == TILE_MASKED && mask_in_lds(st);
        uint2 mr[4];
        const char *mb = reinterpret_cast<const char *>(m_lds + (buf * NW + wave) * MI * 64) + col * 16 + 8 * half;
        lds_pipeline<KSTEPS, kLdsAhead, uint4v>(
            [&](int ks) __attribute__((always_inline)) {
                return *reinterpret_cast<const uint4v *>(kt + k_off[ks & 7] + (ks >> 3) * 256);
            },
            [&](int ks, const uint4v &kf) __attribute__((always_inline)) {
                if constexpr (BF16) {
                    if (ks == 0) mfma_bf16_vacc_first(s, kf, qf[ks]);
                    else mfma_bf16_vacc(s, kf, qf[ks]);
                } else {
                    if (ks == 0) mfma_f16_vacc_first(s, kf, qf[ks]);
                    else mfma_f16_vacc(s, kf, qf[ks]);
                }
                if (HAS_MASK && ks == KSTEPS - 8 && mask_lds_now) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        mr[q4] = *reinterpret_cast<const uint2 *>(mb + ((q4 >> 1) * 64 + (q4 & 1) * 32) * 16);
                }
                if (nfull) {
                    // instruction n at step n * KSTEPS / NDMA
                    static_for<NDMA>([&](auto n_c) __attribute__((always_inline)) {
                        if (ks == (decltype(n_c)::value * KSTEPS) / NDMA) dma_one(n_c);
                    });
                }
            });

        s_wait_after_mfma_vgpr(s);

        // scale and mask (log2 units); this lane holds keys key0 + 8*(r/4) + 4*half + r%4
        if (HAS_MASK && code == TILE_MASKED) {
            if (!mask_lds_now) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int kf = key0 + 8 * q4 + 4 * half;
                    uint16_t m16[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) m16[e] = mrow[min(kf + e, a.kv_len - 1)];
                    mr[q4] = make_uint2(pack2(m16[0], m16[1]), pack2(m16[2], m16[3]));
                }
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t word = e < 2 ? mr[q4].x : mr[q4].y;
                    const uint16_t m16 = (uint16_t)(word >> (16 * (e & 1)));
                    const float mv = MBF16 ? bf16_bits_to_f32(m16) : f16_bits_to_f32(m16);
                    s[4 * q4 + e] = PRESCALE ? fmaf(mv, kLog2e, s[4 * q4 + e]) : fmaf(s[4 * q4 + e], post_scale, mv * kLog2e);
                }
        } else if constexpr (!PRESCALE) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] *= post_scale;
        }
        if (!full_stage) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (key0 + 8 * (r >> 2) + 4 * half + (r & 3) >= a.kv_len) s[r] = -INFINITY;
        }

        // online softmax for this lane's query (16 keys here, 16 in lane ^ 32)
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = max_with_other_half(mx);
        const bool grow = mx > m_run + kRescaleThreshold;
        const float m_new = grow ? mx : m_run;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
        float rowsum = 0.f;
        uint4v pb[2];
        uint4v pl[BF16 ? 2 : 1];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            uint32_t w[4], wl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(s[8 * e + 2 * i] - m_use);
                const float p1 = __builtin_amdgcn_exp2f(s[8 * e + 2 * i + 1] - m_use);
                if constexpr (BF16) pack_p_bf16(p0, p1, w[i], wl[i], rowsum);
                else w[i] = pack_p_f16(p0, p1, rowsum);
            }
            pb[e] = uint4v{w[0], w[1], w[2], w[3]};
            if constexpr (BF16) pl[e] = uint4v{wl[0], wl[1], wl[2], wl[3]};
        }
        rowsum = sum_with_other_half(rowsum);
        l_run = l_run * alpha + rowsum;
        m_run = m_new;
        if (__ballot(grow)) {
#pragma unroll
            for (int db = 0; db < DBLK; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc_o[db][r] = scale_acc(acc_o[db][r], alpha);
        }

        // O^T[d][query] += V^T[d][key] P^T[key][query]; step i: P^T half u = i / DBLK into O block i % DBLK
        lds_pipeline<2 * DBLK, kLdsAhead, uint4v>(
            [&](int i) __attribute__((always_inline)) {
                const int u = i / DBLK, db = i % DBLK;
                const char *p0 = vt + v_off[db & 3] + 64 * (db & ~3) + u * 32 * D;
                return read_tr16_pair(reinterpret_cast<const uint16_t *>(p0),
                                      reinterpret_cast<const uint16_t *>(p0 + 16 * D));
            },
            [&](int i, const uint4v &vf) __attribute__((always_inline)) {
                acc_o[i % DBLK] = mfma32<BF16>(vf, pb[i / DBLK], acc_o[i % DBLK]);
                if constexpr (BF16) acc_o[i % DBLK] = mfma32<BF16>(vf, pl[i / DBLK], acc_o[i % DBLK]);
            });
        buf ^= 1;
        st = nxt;
    }

    // ---- epilogue: O = O^T / l straight from the accumulators; lane (col, half) holds
    // rows d = 32*db + 8*r4 + 4*half + 0..3 of its query's output row
    if (row_ok) {
        const float sc = l_run > 0.f ? 1.f / l_run : 0.f;
        float *orow = a.o + b * a.o_bs + (int64_t)row * a.o_rs + (int64_t)head * a.o_hs + 4 * half;
#pragma unroll
        for (int db = 0; db < DBLK; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                float4v x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc_o[db][4 * r4 + e] * sc;
                *reinterpret_cast<float4v *>(orow + 32 * db + 8 * r4) = x;
            }
    }
}

// One wave classifies TPW consecutive 64-key tiles of one query block: TILE_SKIP
// when every entry is -inf, TILE_OPEN when every entry is zero, else TILE_MASKED.
// The pass also clears the status block and the pair counters the attention pass
// uses.  Only entries of real rows (< rows) and keys (< kv_len) are read.  Grid:
// (ceil(kv_tiles / (4 * TPW)), row_blocks, batch * blk_heads), four waves per
// block.  Several tiles per wave keep more bytes in flight per wave when there are
// waves enough to fill the chip anyway.
template <int TPW>
__global__ __launch_bounds__(256) void classify_kernel(PrefillArgs a, uint8_t *blk) {
    constexpr int kClassifyTiles = TPW;
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < kStatusWords) a.status[threadIdx.x] = 0u;
    if (a.n_pair_cnt > 0) {
        // the pair counters of the attention pass start from zero on every call
        const int64_t nthreads = (int64_t)gridDim.x * gridDim.y * gridDim.z * 256;
        const int64_t tid = (((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) * 256 + threadIdx.x;
        for (int64_t i = tid; i < a.n_pair_cnt; i += nthreads) a.pair_cnt[i] = 0u;
    }
    const int lane = threadIdx.x & 63;
    const int kt0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kClassifyTiles;
    if (kt0 >= a.kv_tiles) return;
    const int rb = blockIdx.y;
    const int hg = blockIdx.z % a.blk_heads;
    const int b = blockIdx.z / a.blk_heads;
    const int slots = a.rows_per_wg * (a.blk_heads == 1 ? 1 : a.heads_per_wg);
    const int h0 = hg * a.heads_per_wg;
    const uint16_t *mbase = (const uint16_t *)a.mask + b * a.m_bs;
    const uint16_t neg_inf = a.mask_bf16 ? 0xFF80u : 0xFC00u;
    // rows_per_wg is a power of two: a slot's (head, row) by shift and mask, not by division
    const int rsh = __builtin_ctz(a.rows_per_wg), rmask = a.rows_per_wg - 1;
    // every mask element of a batch item within 2^31 bytes of its first: 32-bit buffer offsets
    const bool off32 = ((int64_t)(a.n_heads - 1) * a.m_hs + (int64_t)(a.rows - 1) * a.m_rs + a.kv_len) * 2 <
                       ((int64_t)1 << 31);
    uint8_t *out = blk + (((int64_t)b * a.blk_heads + hg) * a.row_blocks + rb) * a.blk_stride;
    auto code_of = [&](bool any_visible, bool any_nonzero) -> uint8_t {
        const bool vis = __ballot(any_visible) != 0;
        const bool nz = __ballot(any_nonzero) != 0;
        return !vis ? TILE_SKIP : (nz ? TILE_MASKED : TILE_OPEN);
    };
    if (a.mask_dma && slots <= 64 && (kt0 + kClassifyTiles) * kTile <= a.kv_len) {
        // all tiles full, at most 64 rows: 8 lanes per 64-key row (8 keys, 16 bytes each),
        // 8 rows per load; the loads of every tile are requested before any is looked at
        const int k8 = 8 * (lane & 7);
        uint4v raw[kClassifyTiles][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (8 * u < slots) {
                const int s_ = min(8 * u + (lane >> 3), slots - 1);
                const int head = h0 + (s_ >> rsh);
                const int row = min(rb * a.rows_per_wg + (s_ & rmask), a.rows - 1);
                const uint16_t *src = mbase + head * a.m_hs + (int64_t)row * a.m_rs + kt0 * kTile + k8;
#pragma unroll
                for (int t = 0; t < kClassifyTiles; ++t) raw[t][u] = *reinterpret_cast<const uint4v *>(src + t * kTile);
            }
        }
#pragma unroll
        for (int t = 0; t < kClassifyTiles; ++t) {
            bool any_visible = false, any_nonzero = false;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s_ = 8 * u + (lane >> 3);
                if (8 * u < slots && s_ < slots && rb * a.rows_per_wg + (s_ & rmask) < a.rows) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint16_t lo = (uint16_t)(raw[t][u][e] & 0xffffu), hi = (uint16_t)(raw[t][u][e] >> 16);
                        any_visible |= lo != neg_inf || hi != neg_inf;
                        any_nonzero |= ((lo | hi) & 0x7fffu) != 0;
                    }
                }
            }
            const uint8_t code = code_of(any_visible, any_nonzero);
            if (lane == 0) out[kt0 + t] = code;
        }
        return;
    }
    for (int kt = kt0; kt < kt0 + kClassifyTiles && kt < a.kv_tiles; ++kt) {
        const int key0 = kt * kTile;
        bool any_visible = false, any_nonzero = false;
        auto see = [&](uint16_t m16) {
            any_visible |= m16 != neg_inf;
            any_nonzero |= (m16 & 0x7fffu) != 0;
        };
        if (a.mask_dma && key0 + kTile <= a.kv_len) {
            // 8 lanes per 64-key row, 8 keys (16 bytes) per lane, 8 rows per load; the 8 loads
            // of 64 rows are requested before any is looked at (addresses clamped to existing
            // rows, the copies not counted), so they share one memory round trip
            const int k8 = key0 + 8 * (lane & 7);
            constexpr int U = 8;
            for (int s0 = 0; s0 < slots; s0 += 8 * U) {
                uint4v raw[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int s = min(s0 + 8 * u + (lane >> 3), slots - 1);
                    const int head = h0 + (s >> rsh);
                    const int row = min(rb * a.rows_per_wg + (s & rmask), a.rows - 1);
                    raw[u] = *reinterpret_cast<const uint4v *>(mbase + head * a.m_hs + (int64_t)row * a.m_rs + k8);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int s = s0 + 8 * u + (lane >> 3);
                    if (s < slots && rb * a.rows_per_wg + (s & rmask) < a.rows) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            see((uint16_t)(raw[u][e] & 0xffffu));
                            see((uint16_t)(raw[u][e] >> 16));
                        }
                    }
                }
            }
        } else {
            // any alignment, or the ragged last tile: one key per lane; 64 rows (32 with 64-bit
            // offsets) are requested before any is looked at.  Keys past kv_len load key kv_len - 1 and slots past the
            // row block load clamped rows: elements of this same tile that are counted anyway,
            // so the ORs below are unchanged and no element needs excluding.  Every lane stays
            // active: the slots' row offsets are computed one per lane, then taken lane by lane
            // as the scalar offset of a buffer load.
            const int key = key0 + lane;
            const int key_c = key < a.kv_len ? key : a.kv_len - 1;
            uint32_t acc_x = 0u, acc_n = 0u;  // OR of (m ^ -inf) and of m over this lane's elements
            if (off32) {
                constexpr int U = 64;
                const __amdgpu_buffer_rsrc_t rsrc =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(mbase), 0, 0x7fffffff, kRawBufferFlags);
                for (int s0 = 0; s0 < slots; s0 += U) {
                    const int sl = min(s0 + (lane & (U - 1)), slots - 1);
                    const uint32_t my_off =
                        (uint32_t)(((int64_t)(h0 + (sl >> rsh)) * a.m_hs +
                                    (int64_t)min(rb * a.rows_per_wg + (sl & rmask), a.rows - 1) * a.m_rs) *
                                   2);
                    uint16_t v[U];
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[u] = __builtin_amdgcn_raw_buffer_load_b16(rsrc, key_c * 2, __builtin_amdgcn_readlane(my_off, u), 0);
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        acc_x |= (uint32_t)(v[u] ^ neg_inf);
                        acc_n |= v[u];
                    }
                }
            } else {
                constexpr int U = 32;
                for (int s0 = 0; s0 < slots; s0 += U) {
                    const int sl = min(s0 + (lane & (U - 1)), slots - 1);
                    const int64_t my_off = (int64_t)(h0 + (sl >> rsh)) * a.m_hs +
                                           (int64_t)min(rb * a.rows_per_wg + (sl & rmask), a.rows - 1) * a.m_rs;
                    const uint32_t off_lo = (uint32_t)my_off, off_hi = (uint32_t)((uint64_t)my_off >> 32);
                    uint16_t v[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const uint64_t off_u = (uint64_t)__builtin_amdgcn_readlane(off_lo, u) |
                                               ((uint64_t)__builtin_amdgcn_readlane(off_hi, u) << 32);
                        v[u] = (mbase + off_u)[key_c];
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        acc_x |= (uint32_t)(v[u] ^ neg_inf);
                        acc_n |= v[u];
                    }
                }
            }
            any_visible = acc_x != 0u;
            any_nonzero = (acc_n & 0x7fffu) != 0u;
        }
        const uint8_t code = code_of(any_visible, any_nonzero);
        if (lane == 0) out[kt] = code;
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
    // eight splits per pass: their (m, l) and partial rows are all requested before any
    // is used, and the running max is rescaled pass by pass
    constexpr int U = 8;
    float mrun = -INFINITY, l = 0.f;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < a.splits; s0 += U) {
        float2 ml[U];
        float4v x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s = min(s0 + u, a.splits - 1);
            ml[u] = a.ml[s * units + unit];
            x[u] = *reinterpret_cast<const float4v *>(a.part + (s * units + unit) * D + 4 * d4);
        }
        float mx = mrun;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s0 + u < a.splits) mx = fmaxf(mx, ml[u].x);
        if (mx == -INFINITY) continue;  // no split so far saw a key
        const float r = mrun == -INFINITY ? 0.f : exp2f(mrun - mx);
        acc *= r;
        l *= r;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s0 + u < a.splits && ml[u].x != -INFINITY) {
                const float w = exp2f(ml[u].x - mx);
                l += w * ml[u].y;
                acc += w * x[u];
            }
        }
        mrun = mx;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int row = unit % a.rows;
    const int64_t bh = unit / a.rows;
    const int head = bh % a.n_heads;
    const int b = bh / a.n_heads;
    *reinterpret_cast<float4v *>(a.o + b * a.o_bs + (int64_t)row * a.o_rs + head * a.o_hs + 4 * d4) = acc * inv;
}

template <int D, int NW, bool BF16, int MASK>
hipError_t launch_nw(const PrefillArgs &a, const PrefillPlan *plan, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)plan->head_groups * plan->row_blocks * a.splits * a.batch));
    if constexpr (BF16) {
        if (!a.q_bf16) {
            // f32 Q against bf16 K/V at head_dim 256 runs two-wave workgroups only (plan_prefill)
            if constexpr (D == 256 && NW == 4) {
                return hipErrorInvalidValue;
            } else {
                hipLaunchKernelGGL((prefill_kernel<D, NW, true, MASK, true>), grid, dim3(64 * NW), 0, stream, a);
                return hipGetLastError();
            }
        }
    }
    hipLaunchKernelGGL((prefill_kernel<D, NW, BF16, MASK, false>), grid, dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

template <int D, bool BF16, int MASK>
hipError_t launch_typed(const PrefillArgs &a, const PrefillPlan *plan, hipStream_t stream) {
    if (plan->waves == 4) return launch_nw<D, 4, BF16, MASK>(a, plan, stream);
    if constexpr (D <= 256) {
        if (plan->waves == 2) return launch_nw<D, 2, BF16, MASK>(a, plan, stream);
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
        err = !has_mask ? launch_typed<D, true, 0>(a, plan, stream)
              : a.mask_bf16 ? launch_typed<D, true, 2>(a, plan, stream)
                            : launch_typed<D, true, 1>(a, plan, stream);
    } else {
        err = !has_mask ? launch_typed<D, false, 0>(a, plan, stream)
              : a.mask_bf16 ? launch_typed<D, false, 2>(a, plan, stream)
                            : launch_typed<D, false, 1>(a, plan, stream);
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
    const bool qsplit = p->q_dtype == ATTN_F32 && p->kv_dtype == ATTN_BF16;
    const int g = p->n_heads / p->n_kv_heads;
    // head_dim 512 with Q in one K/V type (not the f32-Q + bf16-K/V pair): 128-slot
    // workgroups with every wave over the whole head dim, when there are enough of them
    // to fill the chip without splitting the KV range
    plan->wide = 0;
    plan->narrow = 0;
    if (D == 512 && !qsplit) {
        int hpw = 1;  // query heads per workgroup: a power of two dividing g, at most 4 (>= 32 rows)
        for (int d = 2; d <= 4 && d <= g; d *= 2)
            if (g % d == 0) hpw = d;
        const int rpw = 128 / hpw;
        const int64_t wgs = (int64_t)p->batch * ((p->rows + rpw - 1) / rpw) * (p->n_heads / hpw);
        if (wgs >= 256) {
            plan->wide = 1;
            plan->slices = 1;
            plan->slice_dim = D;
            plan->rows_per_wg = rpw;
            plan->heads_per_wg = hpw;
            plan->query_waves = 4;
            plan->waves = 4;
            plan->row_blocks = (p->rows + rpw - 1) / rpw;
            plan->head_groups = p->n_heads / hpw;
            plan->kv_tiles = (p->kv_len + kTile - 1) / kTile;
            plan->blk_stride = (plan->kv_tiles + 3) & ~3;
            plan->splits = 1;
            plan->tiles_per_split = plan->kv_tiles;
            plan->pairing = 0;
            plan->status_offset = 0;
            size_t off = ATTN_PREFILL_STATUS_BYTES;
            const int blk_heads = p->m_hs == 0 ? 1 : plan->head_groups;
            plan->blk_bytes = p->mask_dtype != ATTN_NONE
                                  ? (size_t)p->batch * blk_heads * plan->row_blocks * plan->blk_stride : 0;
            plan->blk_offset = off;
            off = align256(off + plan->blk_bytes);
            plan->ml_offset = plan->ml_bytes = plan->part_offset = plan->part_bytes = 0;
            plan->pair_cnt_offset = plan->pair_cnt_bytes = plan->pair_ml_offset = plan->pair_ml_bytes = 0;
            plan->pair_part_offset = plan->pair_part_bytes = 0;
            plan->workspace_bytes = off;
            return ATTN_OK;
        }
    }
    plan->slices = D > 256 ? 2 : 1;
    plan->slice_dim = D / plan->slices;
    // 128 query slots per workgroup (64 with two head-dim slices); at least 64 slots.
    // 128-slot workgroups at head_dim <= 256 run the eight-wave narrow kernel; 64-slot
    // ones the two-wave prefill_kernel.
    const int max_slots = plan->slices == 1 ? 128 : 64;
    int rpw = pow2_at_least(p->rows < 32 ? p->rows : 32);
    int hpw = 1;  // a power of two, so rows_per_wg * heads_per_wg can reach a multiple of 32
    for (int d = 1; d <= g; d *= 2)
        if (g % d == 0 && rpw * d <= max_slots) hpw = d;
    while ((rpw * hpw) % 64 != 0) rpw *= 2;
    while (rpw * hpw < max_slots && rpw < p->rows) rpw *= 2;
    // fewer, larger workgroups reuse each K/V tile more; below two workgroups per CU
    // (one wave per SIMD each) an unpaired causal tail dominates, so halve them
    // (masked calls pair heavy and light row blocks instead)
    if (plan->slices == 1 && rpw * hpw == 128 && p->mask_dtype == ATTN_NONE &&
        (int64_t)p->batch * (p->n_heads / hpw) * ((p->rows + rpw - 1) / rpw) < 512) {
        if (rpw >= 64) rpw /= 2;
        else if (hpw >= 2) hpw /= 2;
    }
    plan->rows_per_wg = rpw;
    plan->heads_per_wg = hpw;
    plan->narrow = plan->slices == 1 && rpw * hpw == 128;
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
    plan->status_offset = 0;
    size_t off = ATTN_PREFILL_STATUS_BYTES;
    if (p->mask_dtype != ATTN_NONE) {
        const int blk_heads = p->m_hs == 0 ? 1 : plan->head_groups;
        plan->blk_bytes = (size_t)p->batch * blk_heads * plan->row_blocks * plan->blk_stride;
    } else {
        plan->blk_bytes = 0;
    }
    plan->blk_offset = off;
    off = align256(off + plan->blk_bytes);
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
    // paired row blocks (masked calls without a KV split): one partial result per side
    // of every pair, and a counter per pair
    plan->pairing = p->mask_dtype != ATTN_NONE && plan->splits == 1 && plan->row_blocks >= 2;
    if (plan->pairing) {
        const size_t pairs = (size_t)p->batch * plan->head_groups * (plan->row_blocks / 2);
        const size_t slots = (size_t)plan->rows_per_wg * plan->heads_per_wg;
        plan->pair_cnt_offset = off;
        plan->pair_cnt_bytes = 2 * pairs * sizeof(uint32_t);
        off = align256(off + plan->pair_cnt_bytes);
        plan->pair_ml_offset = off;
        plan->pair_ml_bytes = pairs * 2 * slots * sizeof(float2);
        off = align256(off + plan->pair_ml_bytes);
        plan->pair_part_offset = off;
        plan->pair_part_bytes = pairs * 2 * slots * D * sizeof(float);
        off = align256(off + plan->pair_part_bytes);
    } else {
        plan->pair_cnt_offset = plan->pair_cnt_bytes = plan->pair_ml_offset = plan->pair_ml_bytes = 0;
        plan->pair_part_offset = plan->pair_part_bytes = 0;
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
    a.status = (uint32_t *)(w + plan->status_offset);
    a.blk = plan->blk_bytes ? w + plan->blk_offset : nullptr;
    a.ml = plan->splits > 1 ? (float2 *)(w + plan->ml_offset) : nullptr;
    a.part = plan->splits > 1 ? (float *)(w + plan->part_offset) : nullptr;
    a.pairing = plan->pairing;
    a.pair_cnt = plan->pairing ? (uint32_t *)(w + plan->pair_cnt_offset) : nullptr;
    a.pair_ml = plan->pairing ? (float2 *)(w + plan->pair_ml_offset) : nullptr;
    a.pair_part = plan->pairing ? (float *)(w + plan->pair_part_offset) : nullptr;
    a.n_pair_cnt = plan->pairing ? (int)(plan->pair_cnt_bytes / sizeof(uint32_t)) : 0;
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
    // 16-byte mask chunks streamed into LDS need every row start 16-byte aligned
    a.mask_dma = a.mask && (p->m_rs % 8 == 0) && (p->m_hs % 8 == 0) && (p->m_bs % 8 == 0) &&
                 (((uintptr_t)mask & 15u) == 0);
    a.score_scale = p->scale * kLog2e;

    if (a.mask) {
        // four tiles per wave once that still leaves 4096 waves or more
        const int64_t units = (int64_t)plan->kv_tiles * plan->row_blocks * p->batch * a.blk_heads;
        if (units >= 4 * 4096) {
            dim3 grid((plan->kv_tiles + 15) / 16, plan->row_blocks, p->batch * a.blk_heads);
            hipLaunchKernelGGL(classify_kernel<4>, grid, dim3(256), 0, stream, a, (uint8_t *)a.blk);
        } else {
            dim3 grid((plan->kv_tiles + 3) / 4, plan->row_blocks, p->batch * a.blk_heads);
            hipLaunchKernelGGL(classify_kernel<1>, grid, dim3(256), 0, stream, a, (uint8_t *)a.blk);
        }
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    const bool bf16 = p->kv_dtype == ATTN_BF16;
    if (plan->wide) {
        const dim3 grid((unsigned)((int64_t)plan->head_groups * plan->row_blocks * p->batch));
        const int mask = a.mask == nullptr ? 0 : a.mask_bf16 ? 2 : 1;
        if (bf16) {
            if (mask == 0) hipLaunchKernelGGL((wide_kernel<512, true, 0>), grid, dim3(256), 0, stream, a);
            else if (mask == 1) hipLaunchKernelGGL((wide_kernel<512, true, 1>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((wide_kernel<512, true, 2>), grid, dim3(256), 0, stream, a);
        } else {
            if (mask == 0) hipLaunchKernelGGL((wide_kernel<512, false, 0>), grid, dim3(256), 0, stream, a);
            else if (mask == 1) hipLaunchKernelGGL((wide_kernel<512, false, 1>), grid, dim3(256), 0, stream, a);
            else hipLaunchKernelGGL((wide_kernel<512, false, 2>), grid, dim3(256), 0, stream, a);
        }
        return hipGetLastError();
    }
    if (plan->narrow) {
        hipError_t err = launch_narrow_prefill(a, plan, bf16, stream);
        if (err != hipSuccess) return err;
        if (plan->splits > 1) return plan->head_dim == 128 ? launch_combine<128>(a, stream) : launch_combine<256>(a, stream);
        return hipSuccess;
    }
    switch (plan->head_dim) {
    case 128: return launch_for_dim<128>(a, plan, bf16, stream);
    case 256: return launch_for_dim<256>(a, plan, bf16, stream);
    case 512: return launch_for_dim<512>(a, plan, bf16, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
