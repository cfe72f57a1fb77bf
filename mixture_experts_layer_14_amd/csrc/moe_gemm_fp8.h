// moe_gemm_fp8.h -- grouped expert GEMMs for fp8 (OCP e4m3) layers, included
// by moe_gemm.hip only.
//
// Operation (SGLang page "srt/models/deepseek_v2.py": DeepseekV2MLP with fp8
// weight_block_size [128, 128] and a per-token-group-128 fp8 input; the
// SiLU-and-mul output quantised the same way before down_proj):
//   w13:  g/u[r, n] = sum_kb sa[r, kb] * sw[e, n/128, kb] * (qa[r, kb-block] . qw[e, n, kb-block])
//         act = silu(g) * u, then per (row, 128 columns): scale = max(amax,
//         1e-10) / 448, code = e4m3(act / scale);
//   w2:   y[r, h] = w_r * sum_kb sa2[r, kb] * sw2[e, h/128, kb] * (...)
// One k-iteration is exactly one 128-wide scale block: two 32x32x64 fp8 MFMAs
// accumulate the raw block product, which is then scaled and added to the
// fp32 accumulator.  The MFMAs take the weight rows as their first operand,
// so an accumulator lane holds one token and 16 output features of one
// 32-feature block: both scales of a block product are then one value per
// lane and MFMA tile, and the promotion costs one FMA per element (with
// tokens as the first operand every element would need its own scale
// product, which makes the vector ALU, not the matrix core, the limit).
// Staging, swizzle, tile order and the pipeline follow tile_kernel.  The
// per-token A scales and the weight block scales are copied by gathered
// global_load_lds too.  A copy instruction costs the CU's copy path the same
// time whether it moves 4 or 16 bytes a lane, so when the k-blocks of a row
// come in whole groups of SG = 4, each wave copies the scales of a group
// (16 bytes a lane) once per group into a two-slot ring beside the stages;
// otherwise (SG = 1) each stage carries its k-block's scales (4 bytes a
// lane).
#pragma once

#include <type_traits>

#include "moe_gemm_kernels.h"

namespace moe {

template <int BM, int BN, int WM, int WN, int MODE, int SG>
__global__ __launch_bounds__(WM* WN* kWave) void tile_kernel_fp8(GemmArgs g) {
    constexpr int ROWB = 128;                     // one 128-wide k block per stage
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;   // tokens x features per wave
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int SLOTS = ROWB / 16;
    constexpr int RPC = kWave / SLOTS;             // rows per 16-byte copy instruction
    constexpr int COPIES = ROWS / RPC / NW;
    constexpr int SROWS = BM / NW;                 // A-scale rows copied per wave
    // weight-scale blocks per stage: w13 tiles interleave gate and up rows in
    // 32-row blocks (one 128-row scale block of each), w2 tiles hold BN/128
    // consecutive scale blocks
    constexpr int NBS = MODE == kModeW13 ? 2 : BN / 128;
    constexpr bool GROUPED = SG > 1;
    // SG = 1: a stage is the A rows, the B rows, then one 256-byte scale slot
    // per wave (lane l of wave w at byte 4l: the A scale of token w*SROWS+l
    // for l < SROWS; wave 0 also holds the weight block scales at lanes
    // SROWS .. SROWS+NBS-1).
    // SG = 4: a ring slot holds one group's scales by position p, 16 bytes
    // each (the group's 4 scales): A token p for p < BM, weight block scale
    // p-BM for BM <= p < BM+NBS, a copy of token 0's past that.  The copy of
    // wave w covers positions w*SROWS .. w*SROWS+63, so neighbouring waves
    // write some positions twice, always with the same values.
    constexpr int SCALES = GROUPED ? 0 : NW * 256;
    constexpr int STAGE = ROWS * ROWB + SCALES;
    constexpr int SPOS = (NW - 1) * SROWS + kWave;       // positions of a ring slot
    constexpr int RING_SLOT = GROUPED ? (SPOS * 16 + 255) / 256 * 256 : 0;
    constexpr int RING = 2 * RING_SLOT;
    constexpr int PER_STAGE = GROUPED ? COPIES : COPIES + 1;  // copy instructions per wave per stage
    constexpr int LDS_MAX = 160 * 1024;
    constexpr int ROW_W_BYTES = MODE == kModeW2 ? BM * 4 : 0;
    constexpr int STAGES = 4 * STAGE + RING + ROW_W_BYTES <= LDS_MAX ? 4 : 3;
    static_assert(ROWS % (RPC * NW) == 0 && BM % RPC == 0 && BM % NW == 0, "copy split");
    static_assert(SROWS + NBS <= kWave, "scale slots of wave 0");
    static_assert(SG == 1 || SG == 4, "scales per k-block or per group of 4");
    static_assert(!GROUPED || BM + NBS <= SPOS, "ring positions");
    static_assert(!GROUPED || SG >= STAGES - 2, "a group's scale copy lands within the group");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(MODE != kModeW2 || NW * kWave >= BM, "one thread per row weight");
    static_assert(MODE != kModeW13 || (TN == 2 && BN == 256 && WN == 4),
                  "w13 fp8: each wave holds one 32-feature gate/up pair, a block one 128-feature group");
    static_assert(PER_STAGE * (STAGES - 2) + 1 <= 63, "vmcnt immediate range");
    static_assert(MODE != kModeW13 || BM * WN * 4 <= STAGE, "w13 amax exchange fits one stage");
    // one LDS object: the stage buffers, then (w2) the tile's routing
    // weights.  A second __shared__ array would make the compiler wait for
    // every copy in flight before each LDS read of the main loop.
    static_assert(STAGES * STAGE + RING + ROW_W_BYTES <= LDS_MAX, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE + RING + ROW_W_BYTES];
    uint8_t* const ring = smem + STAGES * STAGE;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_index(tid);
    const int wm = wave / WN, wn = wave % WN;

    const TilePos tp = map_block(blockIdx.x, *g.num_tiles, g.n_tiles_n, g.tiles);
    if (!tp.ok) return;
    const Tile tl = g.tiles[tp.m];
    const int n_tile = tp.n;
    const int64_t K = g.Kd;                        // bytes per row (1 byte per value)
    const int nkb = static_cast<int>(K / 128);
    const BSel bw = expert_weights<MODE>(g, tl.expert, 1);
    const bool a_pk = MODE == kModeW2 && g.a_packed;  // w2 reads a packed act

    const uint8_t* src[COPIES];
#pragma unroll
    for (int q = 0; q < COPIES; ++q) {
        const int row = (wave * COPIES + q) * RPC + lane / SLOTS;
        const int chunk = lds_slot<ROWB>(row, lane % SLOTS);
        if (row < BM) {
            int64_t r = tl.row0 + row;
            if (r >= tl.row1) r = tl.row0;
            src[q] = g.A + (MODE == kModeW2 ? act_offset(g, r, chunk * 16, K) : a_source_row<MODE>(g, r) * K + chunk * 16);
        } else {
            src[q] = bw.base + packed_offset(b_weight_row<MODE, BN, 32>(g, bw, n_tile, row - BM), chunk * 16, bw.rb);
        }
    }
    // scale copied by this lane: an A-scale row (lanes < SROWS) or, in wave
    // 0, a weight-scale row (lanes SROWS .. SROWS+NBS-1).  The other lanes
    // copy the wave's first A-scale row into slots nobody reads, so the copy
    // needs no exec mask (a branch would split the loop's scheduling region)
    // (SG = 4: the scales of ring position wave*SROWS + lane)
    const float* ssrc;
    {
        const int p = GROUPED ? wave * SROWS + lane : (lane < SROWS ? wave * SROWS + lane : 0);
        int64_t r = tl.row0 + (p < BM ? p : 0);
        if (r >= tl.row1) r = tl.row0;
        ssrc = g.A_scale + a_source_row<MODE>(g, r) * nkb;
        const int slot = GROUPED ? p - BM : (wave == 0 ? lane - SROWS : -1);
        if (slot >= 0 && slot < NBS) {
            const int rep = MODE == kModeW13 ? slot * 32 : slot * 128;  // a local row of the block
            const int b = static_cast<int>(b_weight_row<MODE, BN, 32>(g, bw, n_tile, rep) / 128);
            ssrc = bw.scale + static_cast<int64_t>(b) * bw.scale_rs;
        }
    }
    // SG = 4: the scales of group grp into ring slot grp % 2
    auto issue_scales = [&](int grp) {
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(ssrc + grp * SG),
            (__attribute__((address_space(3))) void*)(ring + (grp & 1) * RING_SLOT + wave * SROWS * 16), 16, 0, 0);
    };

    // copies q0 .. q1-1 (and, with q1 == COPIES, the scales) of this wave's
    // share of k-block `kit`; past the last k-block the source is clamped to
    // it, keeping the copy count per k-block fixed and the loop branch-free
    auto issue_copies = [&](int kit, int q0, int q1) {
        int kc = kit < nkb ? kit : nkb - 1;
        int sb = (kit % STAGES) * STAGE;
        // opaque per call: with SG = 4 the compiler would otherwise form the
        // sources of all four iterations of a group up front and keep them live
        asm volatile("" : "+s"(kc), "+s"(sb));
        uint8_t* st = smem + sb;
        const int64_t off = static_cast<int64_t>(kc) * ROWB;
#pragma unroll
        for (int q = q0; q < q1; ++q)
            __builtin_amdgcn_global_load_lds(
                // packed B (the later copies) and a packed A advance 16x faster along k
                reinterpret_cast<const void*>(src[q] + (a_pk || (wave * COPIES + q) * RPC >= BM ? off << 4 : off)),
                (__attribute__((address_space(3))) void*)(st + (wave * COPIES + q) * 1024), 16, 0, 0);
        if (!GROUPED && q1 == COPIES)
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(ssrc + kc),
                (__attribute__((address_space(3))) void*)(st + ROWS * ROWB + wave * 256), 4, 0, 0);
    };
    // this wave's copies of all but the STAGES-2 most recent stages landed.
    // Loads complete in order; with SG = 4 a group's scale copy, issued
    // before the stage copies of its first iteration, is one more operation
    // that may stay in flight while that iteration is among the STAGES-2
    // most recent (sub, the iteration's place in its group, < STAGES-2).
    auto wait_later_stages = [&](auto sub_tag) {
        constexpr int sub = decltype(sub_tag)::value;
        constexpr int n = (STAGES - 2) * PER_STAGE + (GROUPED && sub < STAGES - 2 ? 1 : 0);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int lrow = lane % 32, khalf = lane / 32;

    // w2: the tile's routing weights, loaded into a register before the main
    // loop and moved to LDS after it (no copy left in flight to wait for)
    float* row_w = reinterpret_cast<float*>(smem + STAGES * STAGE + RING);
    float my_w = 1.0f;
    if (MODE == kModeW2 && tid < BM) {
        const int64_t r = tl.row0 + tid;
        if (r < tl.row1) my_w = row_weight(g, r);
    }

    // 32 bytes of row r for MFMA step s: 16-byte chunks 4s + 2*khalf, +1
    auto read_frag = [&](const uint8_t* base, int r, int s) {
        const int c0 = s * 4 + khalf * 2;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + r * ROWB + lds_slot<ROWB>(r, c0) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + r * ROWB + lds_slot<ROWB>(r, c0 + 1) * 16);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto read_step = [&](const uint8_t* sA, int s, i32x8 (&fa)[TM], i32x8 (&fb)[TN]) {
        const uint8_t* sB = sA + BM * ROWB;
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = read_frag(sA, wm * WTM + i * 32 + lrow, s);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = read_frag(sB, wn * WTN + j * 32 + lrow, s);
    };
    constexpr int kReads = 2 * (TM + TN), kMfma = TM * TN;
    // blk[i][j]: weight rows (features) x tokens; formats 0/0 are fp8 e4m3
    // with unit (2^0) block scales
    f32x16 blk[TM][TN];
    auto mfma_range = [&](int lo, int hi, const i32x8 (&fa)[TM], const i32x8 (&fb)[TN], bool first) {
#pragma unroll
        for (int m = lo; m < hi; ++m) {
            const f32x16 c = first ? f32x16{} : blk[m / TN][m % TN];
            blk[m / TN][m % TN] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[m % TN], fa[m / TN], c, 0, 0, 0, 127, 0, 127);
        }
    };

    if constexpr (GROUPED) issue_scales(0);
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st) issue_copies(st, 0, COPIES);
    {
        constexpr int n = (STAGES - 2) * PER_STAGE;
        __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    }
    __builtin_amdgcn_s_barrier();
    i32x8 af[2][TM], bfr[2][TN];
    read_step(smem, 0, af[0], bfr[0]);
    const int ngroups = nkb / SG;
    for (int it0 = 0; it0 < nkb; it0 += SG) static_for<SG>([&](auto sub_tag) {
        constexpr int sub = decltype(sub_tag)::value;
        const int it = it0 + sub;
        // each iteration reads its own scales: without this the compiler
        // merges a group's four scale reads and keeps them live across it
        asm volatile("" ::: "memory");
        int sb = (it % STAGES) * STAGE, nb = ((it + 1) % STAGES) * STAGE;
        asm volatile("" : "+s"(sb), "+s"(nb));  // per iteration, as in issue_copies
        const uint8_t* sA = smem + sb;
        // this k-block's scales: the A scale of each of the lane's tokens, the
        // weight scale of each of its 32-feature blocks (read before the
        // barrier below releases the buffer)
        float sa[TM], sw[TN];
        if constexpr (GROUPED) {
            const float* rs = reinterpret_cast<const float*>(ring + ((it0 / SG) & 1) * RING_SLOT);
#pragma unroll
            for (int i = 0; i < TM; ++i) sa[i] = rs[(wm * WTM + i * 32 + lrow) * 4 + sub];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int lr = wn * WTN + j * 32;
                sw[j] = rs[(BM + (MODE == kModeW13 ? (lr / 32) % 2 : lr / 128)) * 4 + sub];
            }
        } else {
            const float* sS = reinterpret_cast<const float*>(sA + ROWS * ROWB);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int t = wm * WTM + i * 32 + lrow;
                sa[i] = sS[(t / SROWS) * 64 + t % SROWS];
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int lr = wn * WTN + j * 32;
                sw[j] = sS[SROWS + (MODE == kModeW13 ? (lr / 32) % 2 : lr / 128)];
            }
        }
        // step 0: step-1 reads, then (first iteration of a group, SG = 4) the
        // next group's scales into the other ring slot, last read in the
        // previous group, and this wave's copies of k-block it+STAGES-1
        // (buffer of k-block it-1, free since the last barrier); the last
        // group copies itself again (same values), keeping the count fixed
        read_step(sA, 1, af[1], bfr[1]);
        constexpr bool SCALE_COPY = GROUPED && sub == 0;
        if constexpr (SCALE_COPY) {
            const int nxt = it0 / SG + 1;
            issue_scales(nxt < ngroups ? nxt : ngroups - 1);
        }
        issue_copies(it + STAGES - 1, 0, COPIES);
        mfma_range(0, kMfma, af[0], bfr[0], true);
        mix_sched<kMfma, kReads, PER_STAGE + (SCALE_COPY ? 1 : 0)>();
        __builtin_amdgcn_sched_barrier(0);
        // step 1, split around the barrier that publishes k-block it+1
        constexpr int H = kMfma / 2;
        mfma_range(0, H, af[1], bfr[1], false);
        __builtin_amdgcn_sched_group_barrier(0x008, H, 0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of stage it landed
        wait_later_stages(sub_tag);
        __builtin_amdgcn_s_barrier();
        read_step(smem + nb, 0, af[0], bfr[0]);
        mfma_range(H, kMfma, af[1], bfr[1], false);
        mix_sched<kMfma - H, kReads, 0>();
        __builtin_amdgcn_sched_barrier(0);
        // promote the block product: one scale per (token tile, feature tile)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const float sc = sa[i] * sw[j];
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(blk[i][j][v], sc, acc[i][j][v]);
            }
    });
    // no copy may still write LDS when the block ends or LDS is reused
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // lane holds token wm*WTM + i*32 + lrow and, of each 32-feature tile j,
    // the features 8*(v/4) + 4*khalf + v%4
    if constexpr (MODE == kModeW13) {
        // act = silu(g) * u; the block's 128 act features are one quantisation
        // group: per-token amax over this wave's 32 features (16 per lane,
        // two lanes per token), then over the WN waves through LDS
        __syncthreads();
        float* red = reinterpret_cast<float*>(smem);  // [BM][WN]
        float act[TM][16];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            float m = 0.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                act[i][v] = glu_act(g, acc[i][0][v], acc[i][1][v]);
                m = fmaxf(m, fabsf(act[i][v]));
            }
            m = fmaxf(m, __shfl_xor(m, 32, kWave));
            if (khalf == 0) red[(wm * WTM + i * 32 + lrow) * WN + wn] = m;
        }
        __syncthreads();
        uint8_t* q = static_cast<uint8_t*>(g.C);
        const int ngroups = g.I / 128;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int lt = wm * WTM + i * 32 + lrow;
            float amax = red[lt * WN];
#pragma unroll
            for (int w = 1; w < WN; ++w) amax = fmaxf(amax, red[lt * WN + w]);
            const float scale = fmaxf(amax, 1e-10f) / 448.0f;
            const int64_t r = tl.row0 + lt;
            if (r < tl.row1) {
                // packed act: columns wn*32 .. +31 lie in one 64-byte piece of the row
                uint8_t* qrow = q + (g.c_packed ? (r >> 4) * (static_cast<int64_t>(g.I) << 4) +
                                                      (static_cast<int64_t>(n_tile) * 2 + (wn >> 1)) * 1024 +
                                                      (r & 15) * 64 + (wn & 1) * 32 + 4 * khalf
                                                : r * g.I + static_cast<int64_t>(n_tile) * 128 + wn * 32 + 4 * khalf);
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    uint32_t word = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        word |= static_cast<uint32_t>(f32_to_e4m3(act[i][4 * b + e] / scale)) << (8 * e);
                    *reinterpret_cast<uint32_t*>(qrow + 8 * b) = word;
                }
                if (wn == 0 && khalf == 0) g.C_scale[r * ngroups + n_tile] = scale;
            }
        }
    } else {
        if (tid < BM) row_w[tid] = my_w;
        __syncthreads();
        uint16_t* y = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int lt = wm * WTM + i * 32 + lrow;
            const int64_t r = tl.row0 + lt;
            if (r >= tl.row1) continue;
            const float w = row_w[lt];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                uint16_t* yrow = y + r * g.N + static_cast<int64_t>(n_tile) * BN + wn * WTN + j * 32 + 4 * khalf;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t lo = static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * b] * w)) |
                                        (static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * b + 1] * w)) << 16);
                    const uint32_t hi = static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * b + 2] * w)) |
                                        (static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * b + 3] * w)) << 16);
                    *reinterpret_cast<uint2*>(yrow + 8 * b) = make_uint2(lo, hi);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// tile_kernel_fp8_256: 256 x 256 fp8 tiles on 8 waves (128 tokens x 64
// features each), for rows whose k blocks come in whole groups of four.
// ---------------------------------------------------------------------------
//
// The 128 x 256 tile above reads, per k block, as many LDS bytes (each wave
// its 64 tokens and 64 features) as its MFMAs take cycles, so LDS and the
// copy path, not the matrix cores, set its pace.  A 256 x 256 tile halves the
// LDS reads per flop (a wave's 128 tokens are reused across its 64 features)
// and cuts the copies per flop by a third; its stage (64 bytes of k of 512
// rows) moves exactly the bytes of the bf16 256 x 256 stage at twice the
// flops.  Its 128 accumulators per lane leave no room for a separate block
// product, so each accumulator is kept in units of the current k block's
// scale product s_kb = sa * sw: before the MFMAs of block kb it is multiplied
// by s_{kb-1} / s_kb, the MFMAs add the raw block product, and the epilogue
// multiplies by the last s.  That is sum_kb s_kb P_kb up to fp32 rounding
// (one extra rounding per k block), with one multiply per element and k
// block, as before.  A k block spans two stages of 64 bytes; four stages fit
// beside a two-slot ring of per-group scales (as above, SG = 4).
// LDS plan of the body below for a BM x BN tile (stages, then the scale
// ring, then the w2 row weights): four stages, or three where four do not
// fit (the 128 x 512 tail tile).
template <int BM, int MODE, int BN_ = 256>
struct Fp8BigShape {
    static constexpr int BN = BN_, NW = 8, ROWB = 64;
    static constexpr int ROWS = BM + BN;
    static constexpr int STAGE = ROWS * ROWB;
    static constexpr int SROWS = BM / NW;
    static constexpr int SPOS = (NW - 1) * SROWS + kWave;
    static constexpr int RING_SLOT = (SPOS * 16 + 255) / 256 * 256;
    static constexpr int RING = 2 * RING_SLOT;
    static constexpr int ROW_W_BYTES = MODE == kModeW2 ? BM * 4 : 0;
    static constexpr int STAGES = 4 * STAGE + RING + ROW_W_BYTES <= 160 * 1024 ? 4 : 3;
    static constexpr int SMEM = STAGES * STAGE + RING + ROW_W_BYTES;
};

// One BM x BN tile (BM x 256 with BM = 256, or 128 for a remainder of at
// most 128 rows: half the copies, LDS reads and MFMAs of a 256-row tile; or
// 128 x 512, a remainder's tile for two n-tiles) of m-tile `tl`, BN-wide
// n-tile `n_tile`; `smem` is the kernel's one LDS array.
template <int BM, int MODE, int BN = 256>
__device__ __forceinline__ void fp8_big_body(const GemmArgs& g, const Tile tl, const int n_tile,
                                             uint8_t* smem) {
    using Shape = Fp8BigShape<BM, MODE, BN>;
    constexpr int WM = 2, WN = 4, NW = WM * WN;
    constexpr int ROWB = Shape::ROWB;              // bytes of k per stage
    constexpr int WTM = BM / WM, WTN = BN / WN;    // tokens x 64 (or 128) features per wave
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int ROWS = Shape::ROWS;
    constexpr int SLOTS = ROWB / 16;
    constexpr int RPC = kWave / SLOTS;             // rows per copy instruction
    constexpr int COPIES = ROWS / RPC / NW;        // copy instructions per wave per stage
    constexpr int STAGE = Shape::STAGE;
    constexpr int STAGES = Shape::STAGES;
    constexpr int SG = 4;                          // k blocks per scale group
    constexpr int SROWS = Shape::SROWS;            // A-scale rows copied per wave
    // weight block scales per k block: BN / 128 weight rows' blocks (w13:
    // half gate, half up blocks, interleaved as the B tile's 32-row blocks)
    constexpr int NBS = BN / 128;
    constexpr int SPOS = Shape::SPOS;
    constexpr int RING_SLOT = Shape::RING_SLOT;
    constexpr int kMfma = TM * TN, HALF = kMfma / 2;
    constexpr int kReads = 2 * (TM + TN);          // ds_read_b128 per stage per wave
    static_assert(ROWS % (RPC * NW) == 0 && BM % RPC == 0, "copy split");
    static_assert(BM + NBS <= SPOS && SROWS + NBS <= kWave, "ring positions");
    static_assert(Shape::SMEM <= 160 * 1024, "LDS budget");
    static_assert(COPIES * (STAGES - 2) + 1 <= 63, "vmcnt immediate range");
    static_assert(MODE != kModeW13 || (TN % 2 == 0 && WN == 4 && 128 % (TN / 2 * 32) == 0),
                  "w13: a wave holds whole gate/up pairs of 32 features inside one 128-column act group");
    static_assert(MODE != kModeW13 || BM * WN * 4 <= STAGE, "w13 amax exchange fits one stage");
    static_assert(HALF % TN == 0, "each half holds whole token blocks");
    uint8_t* const ring = smem + STAGES * STAGE;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_index(tid);
    const int wm = wave / WN, wn = wave % WN;
    const int64_t K = g.Kd;                        // bytes per row
    const int nkb = static_cast<int>(K / 128);
    const int nk = 2 * nkb;                        // stages
    const BSel bw = expert_weights<MODE>(g, tl.expert, 1);
    const bool a_pk = MODE == kModeW2 && g.a_packed;  // w2 reads a packed act

    // source of this lane's 16-byte slot in each of the wave's copies
    const uint8_t* src[COPIES];
#pragma unroll
    for (int q = 0; q < COPIES; ++q) {
        const int row = (wave * COPIES + q) * RPC + lane / SLOTS;
        const int chunk = lds_slot<ROWB>(row, lane % SLOTS);
        if (row < BM) {
            int64_t r = tl.row0 + row;
            if (r >= tl.row1) r = tl.row0;  // ragged tail: copy a valid row, never stored
            src[q] = g.A + (MODE == kModeW2 ? act_offset(g, r, chunk * 16, K) : a_source_row<MODE>(g, r) * K + chunk * 16);
        } else {
            src[q] = bw.base + packed_offset(b_weight_row<MODE, BN, 32>(g, bw, n_tile, row - BM), chunk * 16, bw.rb);
        }
    }
    // scales of ring position wave*SROWS + lane: a token's A scales, a weight
    // block's scales, or (past them) a copy of token 0's
    const float* ssrc;
    {
        const int p = wave * SROWS + lane;
        int64_t r = tl.row0 + (p < BM ? p : 0);
        if (r >= tl.row1) r = tl.row0;
        ssrc = g.A_scale + a_source_row<MODE>(g, r) * nkb;
        const int slot = p - BM;
        if (slot >= 0 && slot < NBS) {
            // a local row of the block (w13: 256-row spans of gate/up 32-row blocks)
            const int rep = MODE == kModeW13 ? (slot / 2) * 256 + (slot % 2) * 32 : slot * 128;
            const int b = static_cast<int>(b_weight_row<MODE, BN, 32>(g, bw, n_tile, rep) / 128);
            ssrc = bw.scale + static_cast<int64_t>(b) * bw.scale_rs;
        }
    }
    auto issue_scales = [&](int grp) {
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(ssrc + grp * SG),
            (__attribute__((address_space(3))) void*)(ring + (grp & 1) * RING_SLOT + wave * SROWS * 16), 16, 0, 0);
    };
    // copies of stage `kit` (64 bytes of k); past the last stage the source is
    // clamped to it, keeping the copy count per stage fixed
    auto issue_copies = [&](int kit) {
        int kc = kit < nk ? kit : nk - 1;
        int sb = (kit % STAGES) * STAGE;
        asm volatile("" : "+s"(kc), "+s"(sb));
        uint8_t* st = smem + sb;
        const int64_t off = static_cast<int64_t>(kc) * ROWB;
#pragma unroll
        for (int q = 0; q < COPIES; ++q)
            __builtin_amdgcn_global_load_lds(
                // packed B (the later copies) and a packed A advance 16x faster along k
                reinterpret_cast<const void*>(src[q] + (a_pk || (wave * COPIES + q) * RPC >= BM ? off << 4 : off)),
                (__attribute__((address_space(3))) void*)(st + (wave * COPIES + q) * 1024), 16, 0, 0);
    };

    // accumulators in units of the current k block's scale product
    f32x16 acc[TM][TN];
    float sprev[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            sprev[i][j] = 1.0f;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
        }

    const int lrow = lane % 32, khalf = lane / 32;
    float* row_w = reinterpret_cast<float*>(smem + STAGES * STAGE + Shape::RING);
    float my_w = 1.0f;
    if (MODE == kModeW2 && tid < BM) {
        const int64_t r = tl.row0 + tid;
        if (r < tl.row1) my_w = row_weight(g, r);
    }

    // 32 bytes of row r of a stage: 16-byte chunks 2*khalf and 2*khalf + 1
    auto read_frag = [&](uint32_t base, int r) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(smem + base + r * ROWB + lds_slot<ROWB>(r, 2 * khalf) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(smem + base + r * ROWB + lds_slot<ROWB>(r, 2 * khalf + 1) * 16);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto read_stage = [&](uint32_t base, i32x8 (&fa)[TM], i32x8 (&fb)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = read_frag(base, wm * WTM + i * 32 + lrow);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = read_frag(base, BM + wn * WTN + j * 32 + lrow);
    };
    // weights first: lane l holds token l%32 of block i and 16 features of
    // the 32 of block j, so both scales are one value per lane and tile
    auto mfma_range = [&](int lo, int hi, const i32x8 (&fa)[TM], const i32x8 (&fb)[TN]) {
#pragma unroll
        for (int m = lo; m < hi; ++m)
            acc[m / TN][m % TN] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb[m % TN], fa[m / TN], acc[m / TN][m % TN], 0, 0, 0, 127, 0, 127);
    };
    // rescale tiles lo..hi-1 to k block kb's units (ratio[m] precomputed)
    float ratio[kMfma], snext[TM][TN];
    // scale products of k block `kb_in_group` of the group in ring slot
    // `slot`, and the ratios to them from the current ones
    auto next_scales = [&](int slot, int kb_in_group) {
        const float* rs = reinterpret_cast<const float*>(ring + slot * RING_SLOT);
        float sa[TM], sw[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) sa[i] = rs[(wm * WTM + i * 32 + lrow) * 4 + kb_in_group];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int lr = wn * WTN + j * 32;
            sw[j] = rs[(BM + (MODE == kModeW13 ? (lr / 256) * 2 + (lr / 32) % 2 : lr / 128)) * 4 + kb_in_group];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                snext[i][j] = sa[i] * sw[j];
                ratio[i * TN + j] = sprev[i][j] * __builtin_amdgcn_rcpf(snext[i][j]);
            }
    };
    auto rescale = [&](int lo, int hi) {
#pragma unroll
        for (int m = lo; m < hi; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[m / TN][m % TN][v] *= ratio[m];
    };
    auto wait_later_stages = [&](auto sub_tag) {
        // stage it+1's copies landed, those of stages it+2 .. it+STAGES-1
        // (and a scale copy issued after stage it+1's) still in flight
        constexpr int sub = decltype(sub_tag)::value;
        constexpr int n = (STAGES - 2) * COPIES + (sub < STAGES - 2 ? 1 : 0);
        __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    };

    issue_scales(0);
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st) issue_copies(st);
    {
        constexpr int n = (STAGES - 2) * COPIES;
        __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    }
    __builtin_amdgcn_s_barrier();
    i32x8 af[2][TM], bfr[2][TN];
    read_stage(0, af[0], bfr[0]);
    next_scales(0, 0);  // k block 0
    const int ngroups = nkb / SG;
    // one group = SG k blocks = 2 * SG stages; sub = the stage's place in it
    for (int it0 = 0; it0 < nk; it0 += 2 * SG) static_for<2 * SG>([&](auto sub_tag) {
        constexpr int sub = decltype(sub_tag)::value;
        constexpr int F = sub & 1;                  // fragment buffer of this stage
        const int it = it0 + sub;
        if constexpr (sub % 2 == 0) {
            // first stage of k block kb: the scale products read during the
            // previous stage become the current ones
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) sprev[i][j] = snext[i][j];
        } else {
            // second stage of k block kb: the next block's scales and ratios
            // (its group's ring slot landed by the barrier that opened this
            // stage: it waited for copies issued after that slot's copy).
            // Past the last block this reads a repeated group whose values
            // are never committed.
            next_scales(sub == 2 * SG - 1 ? ((it0 / (2 * SG)) + 1) & 1 : (it0 / (2 * SG)) & 1,
                        sub == 2 * SG - 1 ? 0 : sub / 2 + 1);
        }
        // the next group's scales (first stage of a group) and this wave's
        // copies of stage it+STAGES-1, into the buffer of stage it-1
        if constexpr (sub == 0) {
            const int nxt = it0 / (2 * SG) + 1;
            issue_scales(nxt < ngroups ? nxt : ngroups - 1);
        }
        issue_copies(it + STAGES - 1);
        if constexpr (sub % 2 == 0) rescale(0, HALF);
        mfma_range(0, HALF, af[F], bfr[F]);
        mix_sched<HALF, 0, COPIES + (sub == 0 ? 1 : 0)>();
        __builtin_amdgcn_sched_barrier(0);
        // next stage's read offsets before the barrier, reads right after it
        uint32_t nb = ((it + 1) % STAGES) * STAGE;
        asm volatile("" : "+v"(nb));
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads landed
        wait_later_stages(std::integral_constant<int, sub % (2 * SG)>{});
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        read_stage(nb, af[F ^ 1], bfr[F ^ 1]);
        if constexpr (sub % 2 == 0) rescale(HALF, kMfma);
        mfma_range(HALF, kMfma, af[F], bfr[F]);
        mix_sched<kMfma - HALF, kReads, 0>();
        __builtin_amdgcn_sched_barrier(0);
    });
    // no copy may still write LDS when the block ends or LDS is reused
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // back to the real scale: acc * s of the last k block
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] *= sprev[i][j];

    // lane holds token wm*WTM + i*32 + lrow and, of each 32-feature tile j,
    // the features 8*(v/4) + 4*khalf + v%4
    if constexpr (MODE == kModeW13) {
        // NP gate/up pairs per wave; GW waves share a 128-column act group
        constexpr int NP = TN / 2, GW = 128 / (NP * 32);
        __syncthreads();
        float* red = reinterpret_cast<float*>(smem);  // [BM][WN]
        float act[TM][NP][16];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            float m = 0.0f;
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    act[i][p][v] = glu_act(g, acc[i][2 * p][v], acc[i][2 * p + 1][v]);
                    m = fmaxf(m, fabsf(act[i][p][v]));
                }
            m = fmaxf(m, __shfl_xor(m, 32, kWave));
            if (khalf == 0) red[(wm * WTM + i * 32 + lrow) * WN + wn] = m;
        }
        __syncthreads();
        uint8_t* q = static_cast<uint8_t*>(g.C);
        const int ngroups_i = g.I / 128;
        const int grp = wn / GW;  // this wave's act group in the tile
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int lt = wm * WTM + i * 32 + lrow;
            float amax = red[lt * WN + grp * GW];
#pragma unroll
            for (int w = 1; w < GW; ++w) amax = fmaxf(amax, red[lt * WN + grp * GW + w]);
            const float scale = fmaxf(amax, 1e-10f) / 448.0f;
            const int64_t r = tl.row0 + lt;
            if (r < tl.row1) {
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    // the pair's 32 act columns lie in one 64-byte piece of the row
                    const int64_t col0 = static_cast<int64_t>(n_tile) * (BN / 2) + (wn * NP + p) * 32;
                    uint8_t* qrow = q + (g.c_packed ? (r >> 4) * (static_cast<int64_t>(g.I) << 4) + (col0 >> 6) * 1024 +
                                                          (r & 15) * 64 + (col0 & 63) + 4 * khalf
                                                    : r * g.I + col0 + 4 * khalf);
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        uint32_t word = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            word |= static_cast<uint32_t>(f32_to_e4m3(act[i][p][4 * b + e] / scale)) << (8 * e);
                        *reinterpret_cast<uint32_t*>(qrow + 8 * b) = word;
                    }
                }
                if (wn % GW == 0 && khalf == 0) g.C_scale[r * ngroups_i + n_tile * (BN / 256) + grp] = scale;
            }
        }
    } else {
        if (tid < BM) row_w[tid] = my_w;
        __syncthreads();
        uint16_t* y = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int lt = wm * WTM + i * 32 + lrow;
            const int64_t r = tl.row0 + lt;
            if (r >= tl.row1) continue;
            const float w = row_w[lt];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                uint16_t* yrow = y + r * g.N + static_cast<int64_t>(n_tile) * BN + wn * WTN + j * 32 + 4 * khalf;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t lo = static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * b] * w)) |
                                        (static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * b + 1] * w)) << 16);
                    const uint32_t hi = static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * b + 2] * w)) |
                                        (static_cast<uint32_t>(f32_to_bf16_bits(acc[i][j][4 * b + 3] * w)) << 16);
                    *reinterpret_cast<uint2*>(yrow + 8 * b) = make_uint2(lo, hi);
                }
            }
        }
    }
}

// 256 x 256 fp8 tiles over the ordinary 256-row tile table: a tile of at
// most 128 rows (an expert's short remainder) runs the 128-row body, inside
// its expert's group, so it shares the group's weight tiles in L2.
template <int MODE>
__global__ __launch_bounds__(8 * kWave) void tile_kernel_fp8_256(GemmArgs g) {
    constexpr int SM = Fp8BigShape<256, MODE>::SMEM, SH = Fp8BigShape<128, MODE>::SMEM;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SM > SH ? SM : SH];
    const TilePos tp = map_block(blockIdx.x, *g.num_tiles, g.n_tiles_n, g.tiles);
    if (!tp.ok) return;
    const Tile tl = g.tiles[tp.m];
    if (tl.row1 - tl.row0 <= 128)
        fp8_big_body<128, MODE>(g, tl, tp.n, smem);
    else
        fp8_big_body<256, MODE>(g, tl, tp.n, smem);
}

// 256 x 256 fp8 tiles with 128 x 512 tail tiles (N a multiple of 512), in
// the schedule and block order of tile_kernel_tail: an expert's remainder of
// at most 128 rows is one 128 x 512 tile per pair of n-tiles, which stages
// 640 rows per 64 bytes of k where two 128 x 256 tiles stage 768, and reads
// a quarter fewer operand bytes from LDS per output column.
template <int MODE>
__global__ __launch_bounds__(8 * kWave) void tile_kernel_fp8_tail(GemmArgs g) {
    constexpr int SM = Fp8BigShape<256, MODE>::SMEM, ST = Fp8BigShape<128, MODE, 512>::SMEM;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SM > ST ? SM : ST];
    const int half = g.n_tiles_n / 2;  // positions per unit
    const int total = *g.num_units * half;
    const int per = (total + 7) / 8;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    if (local >= per) return;
    const int t = xcd * per + local;
    if (t >= total) return;
    const GroupUnit d = g.units[t / half];
    const int w = t - d.first_unit * half;
    const int slot = 2 * d.cnt + d.tail;  // blocks per n-tile pair
    const int pair = w / slot, r = w - pair * slot;
    if (r < 2 * d.cnt)
        fp8_big_body<256, MODE>(g, g.tiles[d.first_tile + r % d.cnt], 2 * pair + r / d.cnt, smem);
    else
        fp8_big_body<128, MODE, 512>(g, g.tiles[d.first_tile + d.cnt], pair, smem);
}

}  // namespace moe
