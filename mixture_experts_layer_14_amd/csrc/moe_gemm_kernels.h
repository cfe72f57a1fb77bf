// moe_gemm_kernels.h -- the two bf16 grouped-GEMM kernel families used by
// moe_gemm.hip (included there only).
//
//  tile_kernel    many rows per expert (prefill): BM x BN block tiles on
//                 32x32x16 bf16 MFMAs, A and B staged through LDS, blocks
//                 ordered so the concurrently resident blocks of one XCD
//                 share weight and activation tiles in that XCD's L2.
//  stream_kernel  few rows per expert (decode): every wave streams its own
//                 weight rows from HBM straight into MFMA operand registers
//                 (no LDS), several k-steps in flight, the 4 waves of a block
//                 splitting K and reducing through LDS at the end.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

typedef __attribute__((ext_vector_type(16))) float f32x16;

enum { kModeW13 = 0, kModeW2 = 1 };

struct GemmArgs {
    const uint8_t* A;           // hidden [T, H] (w13) or act [R, I] (w2)
    const int32_t* sorted_slots;
    const uint8_t* B;           // expert weights [E, N, Kd]
    const uint8_t* B_shared;    // shared expert weights [N, Kd] or null
    const Tile* tiles;
    const int32_t* num_tiles;
    const float* topk_weights;  // w2: routing weight of each slot
    void* C;                    // act [R, I] (w13) or y [R, H] (w2)
    int64_t T;
    int64_t routed_rows;        // T * K
    int32_t topk;
    int32_t Kd;                 // reduction length (elements)
    int32_t N;                  // rows of one expert's weight matrix (2I or H)
    int32_t I;
    int32_t E;
    int32_t n_tiles_n;          // tiles along N
    int32_t max_m_tiles;
    // fp8 layers: per-(row, 128-group) scales of A, 128 x 128 block scales of
    // B, and the per-(row, 128-group) scales written with the w13 output
    const float* A_scale;       // [rows of A, Kd/128]
    const float* B_scale;       // [E, N/128, Kd/128]
    const float* B_shared_scale;  // [N/128, Kd/128]
    float* C_scale;             // w13: [R, I/128]
};

constexpr int kRowBytes = 128;               // bytes of one row per k-iteration
constexpr int kLdsStride = kRowBytes + 16;   // padded row pitch in LDS
constexpr int kChunks = kRowBytes / 16;      // 16-byte chunks per row

// Source row of A for permuted row r: the token of its slot (w13; rows past
// the routed ones belong to the shared expert), or r itself (w2).
template <int MODE>
__device__ __forceinline__ int64_t a_source_row(const GemmArgs& g, int64_t r) {
    if (MODE == kModeW2) return r;
    int64_t src = r >= g.routed_rows ? r - g.routed_rows : g.sorted_slots[r] / g.topk;
    return src < 0 ? 0 : (src >= g.T ? g.T - 1 : src);
}

// Routing weight of permuted row r for the w2 epilogue (shared rows: 1).
__device__ __forceinline__ float row_weight(const GemmArgs& g, int64_t r) {
    return r < g.routed_rows ? g.topk_weights[g.sorted_slots[r]] : 1.0f;
}

// Weight row of local B-tile row `row` for an n-tile of width BN.  w13 tiles
// interleave gate and up rows in blocks of `blk` so that the accumulator
// tile of gate column c and the one of up column c land in the same lanes.
template <int MODE, int BN, int BLK>
__device__ __forceinline__ int64_t b_weight_row(const GemmArgs& g, int n_tile, int row) {
    if (MODE == kModeW2) return static_cast<int64_t>(n_tile) * BN + row;
    const int b = row / BLK, pair = b / 2, up = b % 2;
    const int64_t col = static_cast<int64_t>(n_tile) * (BN / 2) + pair * BLK + row % BLK;
    return up ? g.I + col : col;
}

// Block -> (m-tile, n-tile).  Workgroups are handed to the 8 XCDs round-
// robin, so block b runs on XCD b % 8.  Each XCD takes one contiguous eighth
// of the tile order; inside it, groups of GM m-tiles sweep the n-tiles with
// the m index fastest.  Blocks resident together on an XCD then share their
// A rows (same m-tiles) and weight tiles (same n-tile, same expert) in L2.
struct TilePos {
    int m, n;
    bool ok;
};

__device__ __forceinline__ TilePos map_block(int bid, int num_m, int n_tiles, int GM) {
    TilePos p{0, 0, false};
    const int total = num_m * n_tiles;
    const int per = (total + 7) / 8;
    const int xcd = bid & 7, local = bid >> 3;
    if (local >= per) return p;
    const int t = xcd * per + local;
    if (t >= total) return p;
    const int span = GM * n_tiles;
    const int group = t / span, first = group * GM;
    const int gm = num_m - first < GM ? num_m - first : GM;
    const int w = t - group * span;
    p.m = first + w % gm;
    p.n = w / gm;
    p.ok = true;
    return p;
}

// ---------------------------------------------------------------------------
// tile_kernel (bf16, 32x32x16 MFMA, multi-stage direct-to-LDS pipeline)
// ---------------------------------------------------------------------------
//
// MFMA 32x32x16 bf16 operand layout: lane l holds 8 consecutive k of row
// l%32 (A) or column l%32 (B), k half (l/32).  Accumulator: lane l, value v
// holds row 8*(v/4) + 4*(l/32) + v%4, column l%32.
//
// A k-iteration covers ROWB bytes (ROWB/2 k) of every A row and B row of the
// tile.  Those bytes are copied global -> LDS by global_load_lds_dwordx4
// (no register staging): one instruction moves 1 KiB, lane l filling the
// 16-byte slot l % (ROWB/16) of row l / (ROWB/16).  Slots are XOR-swizzled
// (see lds_slot) so that the MFMA operand reads are free of bank conflicts:
// LDS serves a 128-bit read 16 lanes at a time from 64 four-byte banks, and
// the 16 lanes read 16 consecutive rows at the same logical chunk.  STAGES
// LDS buffers keep the copies of the next STAGES-1 k-iterations in flight
// while the current one multiplies; stage handoff is an explicit vmcnt wait
// plus a bare barrier (a __syncthreads fence would also wait for the copies
// that should stay in flight).
template <int ROWB>
__device__ __forceinline__ int lds_slot(int row, int chunk) {
    // 128-byte rows: even/odd rows fill opposite bank halves, the 8 rows of a
    // parity get 8 slots.  64-byte rows: rows r, r+4, r+8, r+12 share a bank
    // quarter and get 4 slots.
    return ROWB == 128 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 2) & 3);
}

template <int BM, int BN, int WM, int WN, int ROWB, int MODE, int GM>
__global__ __launch_bounds__(WM* WN* kWave) void tile_kernel(GemmArgs g) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int ROWS = BM + BN;                  // rows staged per k-iteration
    constexpr int STAGE = ROWS * ROWB;             // bytes per stage
    constexpr int SLOTS = ROWB / 16;               // 16-byte slots per row
    constexpr int RPC = kWave / SLOTS;             // rows per copy instruction
    constexpr int COPIES = ROWS / RPC / NW;        // copy instructions per wave per stage
    constexpr int KSTEPS = ROWB / 32;              // 16-k MFMA steps per k-iteration
    constexpr int LDS_MAX = 160 * 1024;
#ifndef MOE_TILE_MAX_STAGES
#define MOE_TILE_MAX_STAGES 4
#endif
    constexpr int STAGES_FIT = 4 * STAGE <= LDS_MAX ? 4 : (3 * STAGE <= LDS_MAX ? 3 : 2);
    constexpr int STAGES = STAGES_FIT < MOE_TILE_MAX_STAGES ? STAGES_FIT : MOE_TILE_MAX_STAGES;
    static_assert(ROWB == 64 || ROWB == 128, "row slab of 64 or 128 bytes");
    static_assert(ROWS % (RPC * NW) == 0, "stage rows split evenly over the waves");
    static_assert(BM % RPC == 0, "copy instructions never straddle A and B");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(MODE != kModeW13 || TN % 2 == 0, "w13 wave tile holds gate/up pairs");
    static_assert(COPIES * (STAGES - 2) <= 63, "vmcnt immediate range");
    static_assert(STAGES * STAGE <= LDS_MAX, "LDS budget");
    static_assert(MODE != kModeW2 || NW * kWave >= BM, "one thread per row weight");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / WN, wn = wave % WN;

    const TilePos tp = map_block(blockIdx.x, *g.num_tiles, g.n_tiles_n, GM);
    if (!tp.ok) return;
    const Tile tl = g.tiles[tp.m];
    const int n_tile = tp.n;
    const int64_t eltK = static_cast<int64_t>(g.Kd) * 2;
    const uint8_t* Bexp = tl.expert < g.E
                              ? g.B + static_cast<int64_t>(tl.expert) * g.N * eltK
                              : g.B_shared;

    // source of this lane's 16-byte slot in each of the wave's copies
    const uint8_t* src[COPIES];
#pragma unroll
    for (int q = 0; q < COPIES; ++q) {
        const int row = (wave * COPIES + q) * RPC + lane / SLOTS;
        const int chunk = lds_slot<ROWB>(row, lane % SLOTS);  // the swizzle is an involution
        const uint8_t* base;
        if (row < BM) {
            int64_t r = tl.row0 + row;
            if (r >= tl.row1) r = tl.row0;  // ragged tail: copy a valid row, never stored
            base = g.A + a_source_row<MODE>(g, r) * eltK;
        } else {
            base = Bexp + b_weight_row<MODE, BN, 32>(g, n_tile, row - BM) * eltK;
        }
        src[q] = base + chunk * 16;
    }
    const int nk = static_cast<int>(eltK / ROWB);

    auto issue_stage = [&](int it) {
        uint8_t* dst = smem + (it % STAGES) * STAGE + wave * COPIES * 1024;
        const int64_t off = static_cast<int64_t>(it) * ROWB;
#pragma unroll
        for (int q = 0; q < COPIES; ++q)
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(src[q] + off),
                (__attribute__((address_space(3))) void*)(dst + q * 1024), 16, 0, 0);
    };
    // wait until at most `later` stages of this wave's copies are in flight
    auto wait_copies = [&](int later) {
        if (STAGES >= 4 && later >= 2) {
            constexpr int n = 2 * COPIES;
            __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
        } else if (STAGES >= 3 && later >= 1) {
            constexpr int n = COPIES;
            __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
        } else {
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int lrow = lane % 32, khalf = lane / 32;

    // w2: the tile's routing weights, loaded into a register now so that
    // their dependent loads (slot, then weight) overlap the main loop; they
    // reach LDS only after it, where no copy is left in flight to wait for
    __shared__ float row_w[MODE == kModeW2 ? BM : 1];
    float my_w = 1.0f;
    if (MODE == kModeW2 && tid < BM) {
        const int64_t r = tl.row0 + tid;
        if (r < tl.row1) my_w = row_weight(g, r);
    }
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < nk) issue_stage(st);
    for (int it = 0; it < nk; ++it) {
        // stages it+1 .. it+STAGES-2 may still be in flight
        const int later = min(STAGES - 2, nk - 1 - it);
        wait_copies(later);
        __builtin_amdgcn_s_barrier();
        // every wave has finished reading stage it-1: refill its buffer
        if (it + STAGES - 1 < nk) issue_stage(it + STAGES - 1);

        const uint8_t* sA = smem + (it % STAGES) * STAGE;
        const uint8_t* sB = sA + BM * ROWB;
        // operand fragments double-buffered across the k-steps so the reads
        // of step s+1 are in flight while step s multiplies
        u32x4 af[2][TM], bfr[2][TN];
        auto read_step = [&](int s, u32x4 (&fa)[TM], u32x4 (&fb)[TN]) {
            const int chunk = s * 2 + khalf;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WTM + i * 32 + lrow;
                fa[i] = *reinterpret_cast<const u32x4*>(sA + r * ROWB + lds_slot<ROWB>(r, chunk) * 16);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WTN + j * 32 + lrow;
                fb[j] = *reinterpret_cast<const u32x4*>(sB + r * ROWB + lds_slot<ROWB>(r, chunk) * 16);
            }
        };
        read_step(0, af[0], bfr[0]);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            if (s + 1 < KSTEPS) read_step(s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, af[s & 1][i]), __builtin_bit_cast(bf16x8, bfr[s & 1][j]),
                        acc[i][j], 0, 0, 0);
        }
        // Instruction order of the k-steps above: the first step's operand
        // reads, then for every step its MFMAs with the next step's reads
        // slotted between them, so reads are in flight while the matrix core
        // is busy instead of after it has drained.
        {
            constexpr int kReads = TM + TN, kMfma = TM * TN;
            constexpr int kPaired = kReads < kMfma ? kReads : kMfma;
            constexpr int kRestMfma = kMfma - kPaired, kRestReads = kReads - kPaired;
            __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);       // DS reads, step 0
#pragma unroll
            for (int s = 0; s + 1 < KSTEPS; ++s) {
#pragma unroll
                for (int r = 0; r < kPaired; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
                }
                if (kRestReads > 0) __builtin_amdgcn_sched_group_barrier(0x100, kRestReads, 0);
                if (kRestMfma > 0) __builtin_amdgcn_sched_group_barrier(0x008, kRestMfma, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kMfma, 0);        // last step
        }
        // operand reads of this stage must land before another wave's copy
        // may overwrite it (after the next barrier)
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    }

    if (MODE == kModeW2) {
        if (tid < BM) row_w[tid] = my_w;
        __syncthreads();
    }
    const int ccol = lane % 32;
    const int crow = (lane / 32) * 4;
    if (MODE == kModeW13) {
        uint16_t* act = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int p = 0; p < TN / 2; ++p) {
                const int64_t col = static_cast<int64_t>(n_tile) * (BN / 2) + (wn * (TN / 2) + p) * 32 + ccol;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t r = tl.row0 + wm * WTM + i * 32 + 8 * (v / 4) + crow + (v % 4);
                    if (r < tl.row1)
                        act[r * g.I + col] = f32_to_bf16_bits(silu_mul(acc[i][2 * p][v], acc[i][2 * p + 1][v]));
                }
            }
    } else {
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
                    const int64_t col = static_cast<int64_t>(n_tile) * BN + wn * WTN + j * 32 + ccol;
                    y[r * g.N + col] = f32_to_bf16_bits(acc[i][j][v] * w);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// stream_kernel (bf16, 16x16x32 MFMA, weights straight to registers)
// ---------------------------------------------------------------------------
//
// Block = one m-tile of TM*16 rows x one n-group of NPW 16-column tiles; its
// WAVES waves split the k-steps (64 bytes = 32 k each) evenly.  A lane holds
// 16 bytes of row l%16 at byte (l/16)*16 of the k-step (the 16x16x32 operand
// layout); U k-steps of every operand are loaded before they are consumed.
// For w13 the n-group is NPW/2 gate tiles each followed by its up tile.
template <int TM, int NPW, int WAVES, int MODE, int U>
__global__ __launch_bounds__(WAVES * kWave) void stream_kernel(GemmArgs g) {
    static_assert(MODE != kModeW13 || NPW % 2 == 0, "w13 n-group holds gate/up pairs");
    __shared__ f32x4 red[WAVES][TM][NPW][kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int m_tile = blockIdx.x % g.max_m_tiles;
    const int n_grp = blockIdx.x / g.max_m_tiles;
    if (m_tile >= *g.num_tiles) return;
    const Tile tl = g.tiles[m_tile];
    const int64_t eltK = static_cast<int64_t>(g.Kd) * 2;
    const uint8_t* Bexp = tl.expert < g.E
                              ? g.B + static_cast<int64_t>(tl.expert) * g.N * eltK
                              : g.B_shared;
    const int lrow = lane % 16, lk = (lane / 16) * 16;

    const uint8_t* a_ptr[TM];
    const uint8_t* b_ptr[NPW];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        int64_t r = tl.row0 + i * 16 + lrow;
        if (r >= tl.row1) r = tl.row0;
        a_ptr[i] = g.A + a_source_row<MODE>(g, r) * eltK + lk;
    }
#pragma unroll
    for (int j = 0; j < NPW; ++j)
        b_ptr[j] = Bexp + b_weight_row<MODE, NPW * 16, 16>(g, n_grp, j * 16 + lrow) * eltK + lk;

    f32x4 acc[TM][NPW];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < NPW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // w2: routing weights of the 4 rows per m-subtile this lane stores,
    // loaded up front so the dependent loads overlap the k-loop
    float rw[TM][4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t r = tl.row0 + i * 16 + (lane / 16) * 4 + q;
            rw[i][q] = (MODE == kModeW2 && wave == 0 && r < tl.row1) ? row_weight(g, r) : 1.0f;
        }

    const int ks = static_cast<int>(eltK / 64);
    const int s0 = wave * ks / WAVES, s1 = (wave + 1) * ks / WAVES;
    for (int s = s0; s < s1; s += U) {
        u32x4 a[U][TM], b[U][NPW];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s + u < s1) {
                const int64_t off = static_cast<int64_t>(s + u) * 64;
#pragma unroll
                for (int j = 0; j < NPW; ++j) b[u][j] = *reinterpret_cast<const u32x4*>(b_ptr[j] + off);
#pragma unroll
                for (int i = 0; i < TM; ++i) a[u][i] = *reinterpret_cast<const u32x4*>(a_ptr[i] + off);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s + u < s1) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < NPW; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, a[u][i]), __builtin_bit_cast(bf16x8, b[u][j]),
                            acc[i][j], 0, 0, 0);
            }
        }
    }

    if (WAVES > 1) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < NPW; ++j) red[wave][i][j][lane] = acc[i][j];
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < NPW; ++j) {
                f32x4 sum = red[0][i][j][lane];
#pragma unroll
                for (int w = 1; w < WAVES; ++w) sum += red[w][i][j][lane];
                acc[i][j] = sum;
            }
    }

    const int ccol = lane % 16;
    const int crow = (lane / 16) * 4;
    if constexpr (MODE == kModeW13) {
        uint16_t* act = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int p = 0; p < NPW / 2; ++p) {
            const int64_t col = static_cast<int64_t>(n_grp) * (NPW / 2) * 16 + p * 16 + ccol;
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t r = tl.row0 + i * 16 + crow + q;
                    if (r < tl.row1)
                        act[r * g.I + col] = f32_to_bf16_bits(silu_mul(acc[i][2 * p][q], acc[i][2 * p + 1][q]));
                }
        }
    } else {
        uint16_t* y = static_cast<uint16_t*>(g.C);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = tl.row0 + i * 16 + crow + q;
                if (r >= tl.row1) continue;
                const float w = rw[i][q];
#pragma unroll
                for (int j = 0; j < NPW; ++j) {
                    const int64_t col = static_cast<int64_t>(n_grp) * (NPW * 16) + j * 16 + ccol;
                    y[r * g.N + col] = f32_to_bf16_bits(acc[i][j][q] * w);
                }
            }
    }
}

}  // namespace moe
