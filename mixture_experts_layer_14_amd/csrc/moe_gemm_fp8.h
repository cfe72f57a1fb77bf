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
// fp32 accumulator.  Staging, swizzle and tile order follow tile_kernel; the
// per-row A scales of each k-block ride in the same LDS stage, copied by a
// 4-byte gathered global_load_lds.
#pragma once

#include "moe_gemm_kernels.h"

namespace moe {

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM* WN* kWave) void tile_kernel_fp8(GemmArgs g) {
    constexpr int ROWB = 128;                     // one 128-wide k block per stage
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int ROWS = BM + BN;
    constexpr int SLOTS = ROWB / 16;
    constexpr int RPC = kWave / SLOTS;             // rows per 16-byte copy instruction
    constexpr int COPIES = ROWS / RPC / NW;
    constexpr int SROWS = BM / NW;                 // A-scale rows copied per wave
    constexpr int STAGE = ROWS * ROWB + BM * 4;    // rows, then the A scales
    constexpr int PER_STAGE = COPIES + 1;          // copy instructions per wave per stage
    constexpr int LDS_MAX = 160 * 1024;
    constexpr int STAGES = 3 * STAGE <= LDS_MAX ? 3 : 2;
    static_assert(ROWS % (RPC * NW) == 0 && BM % RPC == 0 && BM % NW == 0 && SROWS <= kWave, "copy split");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(MODE != kModeW2 || NW * kWave >= BM, "one thread per row weight");
    static_assert(MODE != kModeW13 || (TN == 2 && BN == 256 && WN == 4),
                  "w13 fp8: each wave holds one 32-column gate/up pair, a block one 128-column group");
    static_assert(PER_STAGE * (STAGES - 2) <= 63, "vmcnt immediate range");
    // one LDS object: the stage buffers, then (w2) the tile's routing
    // weights.  A second __shared__ array would make the compiler wait for
    // every copy in flight before each LDS read of the main loop.
    constexpr int ROW_W_BYTES = MODE == kModeW2 ? BM * 4 : 0;
    static_assert(STAGES * STAGE + ROW_W_BYTES <= LDS_MAX, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE + ROW_W_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;

    const TilePos tp = map_block(blockIdx.x, *g.num_tiles, g.n_tiles_n, g.tiles);
    if (!tp.ok) return;
    const Tile tl = g.tiles[tp.m];
    const int n_tile = tp.n;
    const int64_t K = g.Kd;                        // bytes per row (1 byte per value)
    const int nkb = static_cast<int>(K / 128);
    const bool shared = tl.expert >= g.E;
    const uint8_t* Bexp = shared ? g.B_shared : g.B + static_cast<int64_t>(tl.expert) * g.N * K;
    const float* Bsc = shared ? g.B_shared_scale
                              : g.B_scale + static_cast<int64_t>(tl.expert) * (g.N / 128) * nkb;

    const uint8_t* src[COPIES];
#pragma unroll
    for (int q = 0; q < COPIES; ++q) {
        const int row = (wave * COPIES + q) * RPC + lane / SLOTS;
        const int chunk = lds_slot<ROWB>(row, lane % SLOTS);
        const uint8_t* base;
        if (row < BM) {
            int64_t r = tl.row0 + row;
            if (r >= tl.row1) r = tl.row0;
            base = g.A + a_source_row<MODE>(g, r) * K;
        } else {
            base = Bexp + b_weight_row<MODE, BN, 32>(g, n_tile, row - BM) * K;
        }
        src[q] = base + chunk * 16;
    }
    // A-scale row copied by this lane (lanes >= SROWS idle)
    const float* ssrc;
    {
        const int row = wave * SROWS + (lane < SROWS ? lane : 0);
        int64_t r = tl.row0 + row;
        if (r >= tl.row1) r = tl.row0;
        ssrc = g.A_scale + a_source_row<MODE>(g, r) * nkb;
    }

    auto issue_stage = [&](int it) {
        uint8_t* st = smem + (it % STAGES) * STAGE;
        const int64_t off = static_cast<int64_t>(it) * ROWB;
#pragma unroll
        for (int q = 0; q < COPIES; ++q)
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(src[q] + off),
                (__attribute__((address_space(3))) void*)(st + (wave * COPIES + q) * 1024), 16, 0, 0);
        if (lane < SROWS)
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(ssrc + it),
                (__attribute__((address_space(3))) void*)(st + ROWS * ROWB + wave * SROWS * 4), 4, 0, 0);
    };
    auto wait_copies = [&](int later) {
        if (STAGES >= 3 && later >= 1) {
            constexpr int n = PER_STAGE;
            __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    };

    // weight-scale row block of each 32-column tile of this wave
    int nblk[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
        nblk[j] = static_cast<int>(b_weight_row<MODE, BN, 32>(g, n_tile, wn * WTN + j * 32) / 128);

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int lrow = lane % 32, khalf = lane / 32;
    const int crow = khalf * 4;

    // w2: the tile's routing weights, loaded into a register before the main
    // loop and moved to LDS after it (no copy left in flight to wait for)
    float* row_w = reinterpret_cast<float*>(smem + STAGES * STAGE);
    float my_w = 1.0f;
    if (MODE == kModeW2 && tid < BM) {
        const int64_t r = tl.row0 + tid;
        if (r < tl.row1) my_w = row_weight(g, r);
    }
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < nkb) issue_stage(st);
    for (int it = 0; it < nkb; ++it) {
        wait_copies(min(STAGES - 2, nkb - 1 - it));
        __builtin_amdgcn_s_barrier();
        if (it + STAGES - 1 < nkb) issue_stage(it + STAGES - 1);

        const uint8_t* sA = smem + (it % STAGES) * STAGE;
        const uint8_t* sB = sA + BM * ROWB;
        const float* sS = reinterpret_cast<const float*>(sA + ROWS * ROWB);
        f32x16 blk[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) blk[i][j][v] = 0.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int c0 = s * 4 + khalf * 2;
            i32x8 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + lrow;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(sA + r * ROWB + lds_slot<ROWB>(r, c0) * 16);
                const u32x4 hi = *reinterpret_cast<const u32x4*>(sA + r * ROWB + lds_slot<ROWB>(r, c0 + 1) * 16);
                af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + lrow;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(sB + r * ROWB + lds_slot<ROWB>(r, c0) * 16);
                const u32x4 hi = *reinterpret_cast<const u32x4*>(sB + r * ROWB + lds_slot<ROWB>(r, c0 + 1) * 16);
                bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    // formats 0/0: both operands fp8 e4m3; unit (2^0) block scales
                    blk[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], blk[i][j],
                                                                                0, 0, 0, 127, 0, 127);
        }
        // scale the block product: acc += blk * sa[row] * sw[n-block]
        float sw[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) sw[j] = Bsc[nblk[j] * nkb + it];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            f32x4 sa4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sa4[q] = *reinterpret_cast<const f32x4*>(sS + wm * WTM + i * 32 + 8 * q + crow);
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[i][j][v] = fmaf(blk[i][j][v], sa4[v / 4][v % 4] * sw[j], acc[i][j][v]);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): reads done before the buffer is refilled
    }

    const int ccol = lane % 32;
    if constexpr (MODE == kModeW13) {
        // act = silu(g) * u; the block's 128 act columns are one quantisation
        // group: per-row amax over this wave's 32 columns (lanes of equal
        // khalf), then over the 4 waves of the row band through LDS
        __syncthreads();
        float* red = reinterpret_cast<float*>(smem);  // [BM][WN]
        float act[TM][16];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                act[i][v] = silu_mul(acc[i][0][v], acc[i][1][v]);
                float m = fabsf(act[i][v]);
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
                if (ccol == 0) red[(wm * WTM + i * 32 + 8 * (v / 4) + crow + (v % 4)) * WN + wn] = m;
            }
        __syncthreads();
        uint8_t* q = static_cast<uint8_t*>(g.C);
        const int64_t col = static_cast<int64_t>(n_tile) * 128 + wn * 32 + ccol;
        const int ngroups = g.I / 128;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int lr = wm * WTM + i * 32 + 8 * (v / 4) + crow + (v % 4);
                float amax = red[lr * WN];
#pragma unroll
                for (int w = 1; w < WN; ++w) amax = fmaxf(amax, red[lr * WN + w]);
                const float scale = fmaxf(amax, 1e-10f) / 448.0f;
                const int64_t r = tl.row0 + lr;
                if (r < tl.row1) {
                    q[r * g.I + col] = f32_to_e4m3(act[i][v] / scale);
                    if (wn == 0 && ccol == 0) g.C_scale[r * ngroups + n_tile] = scale;
                }
            }
    } else {
        if (tid < BM) row_w[tid] = my_w;
        __syncthreads();
        uint16_t* y = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int lr = wm * WTM + i * 32 + 8 * (v / 4) + crow + (v % 4);
                const int64_t r = tl.row0 + lr;
                if (r >= tl.row1) continue;
                const float w = row_w[lr];
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t c = static_cast<int64_t>(n_tile) * BN + wn * WTN + j * 32 + ccol;
                    y[r * g.N + c] = f32_to_bf16_bits(acc[i][j][v] * w);
                }
            }
    }
}

}  // namespace moe
