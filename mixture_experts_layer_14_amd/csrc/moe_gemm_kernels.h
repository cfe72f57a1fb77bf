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

#include <utility>

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {


enum { kModeW13 = 0, kModeW2 = 1 };

struct GemmArgs {
    const uint8_t* A;           // hidden [T, H] (w13) or act [R, I] (w2)
    const int32_t* sorted_slots;
    const uint8_t* B;           // expert weights [E, N, Kd], each matrix packed
    const uint8_t* B_shared;    // shared expert weights [N, Kd] packed, or null
    const Tile* tiles;
    const int32_t* num_tiles;
    const GroupUnit* units;     // tile_kernel_tail: group of each unit of positions
    const int32_t* num_units;
    const int32_t* split;       // tile_kernel_ksplit: [split m-tiles, their first row]
    const float* topk_weights;  // w2: routing weight of each slot
    void* C;                    // act [R, I] (w13) or y [R, H] (w2)
    int64_t T;
    int64_t routed_rows;        // T * K
    int32_t topk;
    int32_t Kd;                 // reduction length (elements)
    int32_t N;                  // rows of one expert's weight matrix (2I or H)
    int32_t I;
    int32_t Is;                 // intermediate size of the shared expert (slices * I)
    int32_t E;
    int32_t n_tiles_n;          // tiles along N
    int32_t max_m_tiles;
    // fp8 layers: per-(row, 128-group) scales of A, 128 x 128 block scales of
    // B, and the per-(row, 128-group) scales written with the w13 output
    const float* A_scale;       // [rows of A, Kd/128]
    const float* B_scale;       // [E, N/128, Kd/128]
    const float* B_shared_scale;  // [N/128, Kd/128]
    float* C_scale;             // w13: [R, I/128]
    // w2 split over K: ksplit parts, part p writing y + p * part_stride
    int32_t ksplit;
    int64_t part_stride;
    // activation variants of the w13 epilogue: gated (silu_a(g) * u with g
    // capped at act_limit and u clamped to +-act_limit; +inf: no clamp) or
    // silu_a(h) of a single projection, silu_a(z) = z * sigmoid(act_alpha z);
    // weight_in: the w13 output of a routed row is scaled by its routing
    // weight (= the weight applied to the expert input, the MLP being linear
    // up to the activation) and the w2 epilogue then adds rows unweighted
    int32_t gated;
    int32_t weight_in;
    float act_alpha;
    float act_limit;
    // act in the packed layout of the weights (moe_forward's own act buffer,
    // tile kernels only): written so by w13 (c_packed), read so by w2
    // (a_packed), every 16-row x 64-byte piece one contiguous KiB
    int32_t a_packed;
    int32_t c_packed;
};

constexpr int kRowBytes = 128;               // bytes of one row per k-iteration
constexpr int kLdsStride = kRowBytes + 16;   // padded row pitch in LDS
constexpr int kChunks = kRowBytes / 16;      // 16-byte chunks per row

// Source row of A for permuted row r: the token of its slot (w13; rows past
// the routed ones belong to the shared expert's slices, T rows each), or r
// itself (w2).
template <int MODE>
__device__ __forceinline__ int64_t a_source_row(const GemmArgs& g, int64_t r) {
    if (MODE == kModeW2) return r;
    int64_t src = r >= g.routed_rows ? (r - g.routed_rows) % g.T : g.sorted_slots[r] / g.topk;
    return src < 0 ? 0 : (src >= g.T ? g.T - 1 : src);
}

// Weights are stored packed: a matrix of `rows` rows of `row_bytes` bytes
// is laid out as [rows/16][row_bytes/64][16][64], so 16 consecutive rows x
// 64 bytes of k form one contiguous KiB.  That is exactly what one 16-row
// copy instruction or one 16x16 MFMA k-step reads, turning 16 short
// strided row pieces into one sequential burst.  Byte offset of (row, byte):
__device__ __forceinline__ int64_t packed_offset(int64_t row, int64_t byte, int64_t row_bytes) {
    return (row >> 4) * (row_bytes << 4) + (byte >> 6) * 1024 + (row & 15) * 64 + (byte & 63);
}

// Byte offset of (row r, byte `byte`) of a w2 A operand (act): packed or
// row-major with `row_bytes` per row.
__device__ __forceinline__ int64_t act_offset(const GemmArgs& g, int64_t r, int64_t byte, int64_t row_bytes) {
    return g.a_packed ? packed_offset(r, byte, row_bytes) : r * row_bytes + byte;
}

// Element index of (row r, column c) of the bf16 act written by w13
// (32 elements per 64-byte piece).
__device__ __forceinline__ int64_t act_store_index(const GemmArgs& g, int64_t r, int64_t c) {
    return g.c_packed ? (r >> 4) * (static_cast<int64_t>(g.I) << 4) + (c >> 5) * 512 + (r & 15) * 32 + (c & 31)
                      : r * g.I + c;
}

// Routing weight of permuted row r for the w2 epilogue (shared rows, and
// every row when the weight went into the expert input: 1).
__device__ __forceinline__ float row_weight(const GemmArgs& g, int64_t r) {
    return (!g.weight_in && r < g.routed_rows) ? g.topk_weights[g.sorted_slots[r]] : 1.0f;
}

// Routing weight of permuted row r on the input side (w13 with weight_in).
__device__ __forceinline__ float in_weight(const GemmArgs& g, int64_t r) {
    return r < g.routed_rows ? g.topk_weights[g.sorted_slots[r]] : 1.0f;
}

// The w13 activations: silu_a(z) = z * sigmoid(a z), evaluated as
// z * rcp(1 + 2^(-a log2(e) z)) with the hardware exp2 and reciprocal (each
// within 1 ulp; the result is rounded to bf16 or kept as fp32 far inside the
// tolerances).  For z -> -inf the reciprocal of inf is 0, for z -> +inf the
// exponential is 0: no overflow path.  The clamp is one med3 per operand
// (act_limit = +inf: no clamp).
__device__ __forceinline__ float silu_a(float z, float a) {
    const float e = __builtin_amdgcn_exp2f(-a * 1.44269504088896341f * z);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float glu_act(const GemmArgs& g, float gate, float up) {
    gate = __builtin_amdgcn_fmed3f(gate, -__builtin_huge_valf(), g.act_limit);
    up = __builtin_amdgcn_fmed3f(up, -g.act_limit, g.act_limit);
    return silu_a(gate, g.act_alpha) * up;
}

// The weight matrix a tile multiplies with: routed expert e's, or slice j of
// the shared expert (expert == E + j).  The shared expert's intermediate
// dimension Is is cut into I-wide slices; the down projection sums over it,
// so slice j is an MLP of its own: gate rows [jI, (j+1)I) and up rows
// [Is + jI, Is + (j+1)I) of the [2Is, H] w13, columns [jI, (j+1)I) of the
// [H, Is] w2.  Element (row, byte) of the matrix is at
// base + packed_offset(row, byte, rb); gate0 / up0 are the first rows of the
// gate and up blocks (w13); scale points at the fp8 block scale of block row
// 0, k block 0, with scale_rs scales per block row.
struct BSel {
    const uint8_t* base;
    int64_t rb;
    int32_t gate0, up0;
    const float* scale;
    int32_t scale_rs;
};

template <int MODE>
__device__ __forceinline__ BSel expert_weights(const GemmArgs& g, int expert, int elt) {
    const int64_t rb = static_cast<int64_t>(g.Kd) * elt;
    const int kb = g.Kd / 128;  // k blocks of a row (fp8 scales)
    BSel s;
    if (expert < g.E) {
        s.base = g.B + static_cast<int64_t>(expert) * g.N * rb;
        s.rb = rb;
        s.gate0 = 0;
        s.up0 = g.I;
        s.scale = g.B_scale + static_cast<int64_t>(expert) * (g.N / 128) * kb;
        s.scale_rs = kb;
    } else if (MODE == kModeW13) {
        const int j = expert - g.E;
        s.base = g.B_shared;
        s.rb = rb;
        s.gate0 = j * g.I;
        s.up0 = g.Is + j * g.I;
        s.scale = g.B_shared_scale;
        s.scale_rs = kb;
    } else {
        // a k offset of j*I*elt bytes is (j*I*elt / 64) KiB blocks of the
        // packed layout (I*elt is a multiple of 64)
        const int j = expert - g.E;
        s.base = g.B_shared + static_cast<int64_t>(j) * g.I * elt * 16;
        s.rb = static_cast<int64_t>(g.Is) * elt;
        s.gate0 = 0;
        s.up0 = 0;
        s.scale = g.B_shared_scale + j * (g.I / 128);
        s.scale_rs = g.Is / 128;
    }
    return s;
}

// Weight row of local B-tile row `row` for an n-tile of width BN.  w13 tiles
// interleave gate and up rows in blocks of `blk` so that the accumulator
// tile of gate column c and the one of up column c land in the same lanes.
template <int MODE, int BN, int BLK>
__device__ __forceinline__ int64_t b_weight_row(const GemmArgs& g, const BSel& s, int n_tile, int row) {
    if (MODE == kModeW2) return static_cast<int64_t>(n_tile) * BN + row;
    if (!g.gated) return s.gate0 + static_cast<int64_t>(n_tile) * BN + row;
    const int b = row / BLK, pair = b / 2, up = b % 2;
    const int64_t col = static_cast<int64_t>(n_tile) * (BN / 2) + pair * BLK + row % BLK;
    return (up ? s.up0 : s.gate0) + col;
}

// Block -> (m-tile, n-tile).  Workgroups are handed to the 8 XCDs round-
// robin, so block b runs on XCD b % 8.  Each XCD takes one contiguous eighth
// of the tile order; inside it, groups of m-tiles of one expert (at most 8,
// so an expert with many m-tiles forms several groups) sweep the n-tiles
// with the m index fastest.  Blocks resident together on an XCD then share
// their A rows (same m-tiles) and weight tiles (same n-tile of the same
// expert) in L2, and each weight tile is streamed once per group.
struct TilePos {
    int m, n;
    bool ok;
};

__device__ __forceinline__ TilePos map_block(int bid, int num_m, int n_tiles, const Tile* tiles) {
    TilePos p{0, 0, false};
    const int total = num_m * n_tiles;
    const int per = (total + 7) / 8;
    const int xcd = bid & 7, local = bid >> 3;
    if (local >= per) return p;
    const int t = xcd * per + local;
    if (t >= total) return p;
    // group g (m-tiles first .. first+cnt-1) owns tile-order positions
    // [first * n_tiles, (first + cnt) * n_tiles), so t / n_tiles is one of
    // its m-tiles and that tile names the group
    const int grp = tiles[t / n_tiles].group;
    const int first = grp >> 8, cnt = grp & 255;
    const int w = t - first * n_tiles;
    p.m = first + w % cnt;
    p.n = w / cnt;
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
// LDS buffers keep the copies of STAGES-2 later k-iterations in flight while
// one multiplies; stage handoff is an explicit vmcnt wait plus a bare
// barrier (a __syncthreads fence would also wait for the copies that should
// stay in flight), one per k-iteration.
template <int ROWB>
__device__ __forceinline__ int lds_slot(int row, int chunk) {
    // 128-byte rows: even/odd rows fill opposite bank halves, the 8 rows of a
    // parity get 8 slots.  64-byte rows: rows r, r+4, r+8, r+12 share a bank
    // quarter and get 4 slots.
    return ROWB == 128 ? chunk ^ ((row >> 1) & 7) : chunk ^ ((row >> 2) & 3);
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1 (compile-time
// loop index, so per-iteration counts can feed scheduling templates).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Scheduling groups for a region that holds LDS reads, then copies into
// LDS (the compiler keeps LDS reads ahead of copies into LDS), then MFMAs:
// the first MFMAs take two reads each so the reads land early, the
// remaining ones share the copies.
template <int MFMAS, int READS, int VMEM, int I = 0>
__device__ __forceinline__ void mix_sched() {
    constexpr int RSLOTS = (READS + 1) / 2 < MFMAS ? (READS + 1) / 2 : MFMAS;
    constexpr int VSLOTS = MFMAS - RSLOTS;
    if constexpr (I < MFMAS) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if constexpr (I < RSLOTS) {
            constexpr int rd = READS - 2 * I >= 2 ? 2 : READS - 2 * I;
            __builtin_amdgcn_sched_group_barrier(0x100, rd, 0);  // DS read
        } else {
            constexpr int vper = (VMEM + VSLOTS - 1) / VSLOTS;
            constexpr int v0 = vper * (I - RSLOTS);
            constexpr int vm = VMEM - v0 >= vper ? vper : (VMEM - v0 > 0 ? VMEM - v0 : 0);
            if constexpr (vm > 0) __builtin_amdgcn_sched_group_barrier(0x020, vm, 0);  // copies
        }
        mix_sched<MFMAS, READS, VMEM, I + 1>();
    } else {
        constexpr int rleft = READS - 2 * RSLOTS;
        constexpr int vleft = VSLOTS > 0 ? 0 : VMEM;
        if constexpr (rleft > 0) __builtin_amdgcn_sched_group_barrier(0x100, rleft, 0);
        if constexpr (vleft > 0) __builtin_amdgcn_sched_group_barrier(0x020, vleft, 0);
    }
}

// LDS plan of a BM x BN tile with ROWB-byte row slabs: as many stages (4, 3
// or 2) as fit in the 160 KiB beside the tile's BM routing weights.
template <int BM, int BN, int ROWB>
struct TileShape {
    static constexpr int ROWS = BM + BN;        // rows staged per k-iteration
    static constexpr int STAGE = ROWS * ROWB;   // bytes per stage
    static constexpr int LDS_MAX = 160 * 1024;
    static constexpr int LDS_STAGES = LDS_MAX - BM * 4;
    static constexpr int STAGES = 4 * STAGE <= LDS_STAGES ? 4 : (3 * STAGE <= LDS_STAGES ? 3 : 2);
    static constexpr int SMEM = STAGES * STAGE + BM * 4;
};

// Main loop of a tile: the guarded one (MFMAs of 32-row blocks past the
// tile's rows skipped) only for tiles with fewer than BM rows, always, or
// never (every MFMA runs; rows past the tile are computed and not stored).
enum { kLoopAuto = 0, kLoopGuarded = 1, kLoopFull = 2 };

// One BM x BN output tile (m-tile `tl`, n-tile `n_tile`, K part `kpart` of
// `nparts`) on WM x WN waves; `smem` is the kernel's one LDS array, at least
// TileShape::SMEM bytes.
template <int BM, int BN, int WM, int WN, int ROWB, int MODE, int LOOP>
__device__ __forceinline__ void tile_body(const GemmArgs& g, const Tile tl, const int n_tile,
                                          const int kpart, const int nparts, uint8_t* smem) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    using Shape = TileShape<BM, BN, ROWB>;
    constexpr int ROWS = Shape::ROWS;
    constexpr int STAGE = Shape::STAGE;
    constexpr int SLOTS = ROWB / 16;               // 16-byte slots per row
    constexpr int RPC = kWave / SLOTS;             // rows per copy instruction
    // Copy instructions per wave per stage.  Every wave takes an equal share
    // of the stage's rows when they split evenly; otherwise (320 x 256: 36
    // copies for 8 waves, 192 x 256: 28) the first half of the waves copy the
    // A rows (CA each) and the second half the B rows (CB each), and each
    // half runs a main loop of its own with its own copy count.
    constexpr bool SPLIT = ROWS % (RPC * NW) != 0;
    constexpr int CA = SPLIT ? BM / RPC / (NW / 2) : ROWS / RPC / NW;
    constexpr int CB = SPLIT ? BN / RPC / (NW / 2) : CA;
    constexpr int COPIES = CA > CB ? CA : CB;      // the larger share
    constexpr int KSTEPS = ROWB / 32;              // 16-k MFMA steps per k-iteration
    constexpr int LDS_MAX = Shape::LDS_MAX;
    constexpr int STAGES = Shape::STAGES;
    static_assert(ROWB == 64 || ROWB == 128, "row slab of 64 or 128 bytes");
    static_assert(!SPLIT || (NW % 2 == 0 && BM % (RPC * NW / 2) == 0 && BN % (RPC * NW / 2) == 0),
                  "stage rows split evenly over the waves, or A and B rows over two halves of them");
    static_assert(BM % RPC == 0, "copy instructions never straddle A and B");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(MODE != kModeW13 || TN % 2 == 0, "w13 wave tile holds gate/up pairs");
    static_assert(KSTEPS % 2 == 0, "a stage ends on fragment buffer 1");
    static_assert(COPIES * (STAGES - 2) <= 63, "vmcnt immediate range");
    static_assert(NW * kWave >= BM, "one thread per row weight");
    // one LDS object: the stage buffers, then the tile's routing weights
    // (w2, or w13 with the weight on the input).  A second __shared__ array
    // would make the compiler wait for every copy in flight before each LDS
    // read of the main loop.
    constexpr int ROW_W_BYTES = BM * 4;
    static_assert(STAGES * STAGE + ROW_W_BYTES <= LDS_MAX, "LDS budget");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_index(tid);
    const int wm = wave / WN, wn = wave % WN;
    const int64_t eltK = static_cast<int64_t>(g.Kd) * 2;
    const BSel bw = expert_weights<MODE>(g, tl.expert, 2);

    // first stage row of this wave's copy q (wave-uniform); with SPLIT the
    // A half of the waves copies rows [0, BM), the B half rows [BM, ROWS)
    const bool a_wave = !SPLIT || wave < NW / 2;
    auto copy_row0 = [&](int q) {
        if constexpr (SPLIT) return a_wave ? (wave * CA + q) * RPC : BM + ((wave - NW / 2) * CB + q) * RPC;
        return (wave * COPIES + q) * RPC;
    };
    // source of this lane's 16-byte slot in each of the wave's copies (with
    // SPLIT, a wave's copies past its own count are never issued; they alias
    // its first)
    const uint8_t* src[COPIES];
#pragma unroll
    for (int q = 0; q < COPIES; ++q) {
        const int row = copy_row0(q < (a_wave ? CA : CB) ? q : 0) + lane / SLOTS;
        const int chunk = lds_slot<ROWB>(row, lane % SLOTS);  // the swizzle is an involution
        if (row < BM) {
            int64_t r = tl.row0 + row;
            if (r >= tl.row1) r = tl.row0;  // ragged tail: copy a valid row, never stored
            src[q] = g.A + (MODE == kModeW2 ? act_offset(g, r, chunk * 16, eltK)
                                            : a_source_row<MODE>(g, r) * eltK + chunk * 16);
        } else {
            src[q] = bw.base + packed_offset(b_weight_row<MODE, BN, 32>(g, bw, n_tile, row - BM), chunk * 16, bw.rb);
        }
    }
    // this block's k-iterations: part kpart of the nk_all of a full row
    const int nk_all = static_cast<int>(eltK / ROWB);
    const int k_first = kpart * nk_all / nparts;
    const int nk = (kpart + 1) * nk_all / nparts - k_first;
    // bytes per k-iteration along a source row: ROWB in a row-major A,
    // ROWB/64 KiB-blocks in the packed B (whose copies are the later ones)
    // and in a packed A
    const bool a_pk = MODE == kModeW2 && g.a_packed;
    auto kstep_shift = [&](int q) { return a_pk || copy_row0(q) >= BM ? 4 : 0; };
#pragma unroll
    for (int q = 0; q < COPIES; ++q) src[q] += (static_cast<int64_t>(k_first) * ROWB) << kstep_shift(q);

    // copies q0 .. q1-1 of this wave's share of k-iteration `kit`; past the
    // last k-iteration the source is clamped to it (a redundant in-bounds
    // copy into a buffer nobody reads again keeps the copy count per
    // k-iteration fixed and the loop free of branches)
    const int copy_dst = copy_row0(0) * ROWB;  // RPC rows of ROWB bytes: 1 KiB per copy
    auto issue_copies = [&](int kit, int q0, int q1) {
        uint8_t* dst = smem + (kit % STAGES) * STAGE + copy_dst;
        const int64_t off = static_cast<int64_t>(kit < nk ? kit : nk - 1) * ROWB;
#pragma unroll
        for (int q = q0; q < q1; ++q)
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(src[q] + (off << kstep_shift(q))),
                (__attribute__((address_space(3))) void*)(dst + q * 1024), 16, 0, 0);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    const int lrow = lane % 32, khalf = lane / 32;

    // the tile's routing weights (w2, or w13 with the weight on the input),
    // loaded into a register now so that their dependent loads (slot, then
    // weight) overlap the main loop; they reach LDS only after it, where no
    // copy is left in flight to wait for
    float* row_w = reinterpret_cast<float*>(smem + STAGES * STAGE);
    const bool use_w = MODE == kModeW2 || g.weight_in;
    float my_w = 1.0f;
    if (use_w && tid < BM) {
        const int64_t r = tl.row0 + tid;
        if (r < tl.row1) my_w = MODE == kModeW2 ? row_weight(g, r) : in_weight(g, r);
    }
    // Operand fragments are double-buffered across k-steps, and across
    // stages too: the first k-step of stage it+1 is read from LDS while the
    // last MFMAs of stage it run, so the matrix core never waits for a
    // stage's first reads.  The barrier that publishes stage it+1 sits in the
    // middle of stage it's last k-step; after it every wave has finished
    // reading stage it, whose buffer then takes the copies of stage
    // it+STAGES.
    // LDS byte offsets of this lane's operand reads in k-step s of a stage:
    // a 32-row block's swizzle depends on the lane alone, so block i (j) of
    // the wave tile is i (j) * 32 rows further
    auto a_lane = [&](int s) -> uint32_t {
        const int r = wm * WTM + lrow;
        return r * ROWB + lds_slot<ROWB>(r, s * 2 + khalf) * 16;
    };
    auto b_lane = [&](int s) -> uint32_t {
        const int r = wn * WTN + lrow;
        return BM * ROWB + r * ROWB + lds_slot<ROWB>(r, s * 2 + khalf) * 16;
    };
    auto read_at = [&](uint32_t pa, uint32_t pb, u32x4 (&fa)[TM], u32x4 (&fb)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[i] = *reinterpret_cast<const u32x4*>(smem + pa + i * 32 * ROWB);
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[j] = *reinterpret_cast<const u32x4*>(smem + pb + j * 32 * ROWB);
    };
    constexpr int kReads = TM + TN, kMfma = TM * TN;
    // this wave's copies (NC per stage) of all but the STAGES-2 most recent
    // stages landed
    auto wait_later_stages = [&](auto nc_tag) {
        constexpr int n = (STAGES - 2) * decltype(nc_tag)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    };
    // A ragged last tile of an expert skips the MFMAs of 32-row blocks that
    // lie wholly past its rows (copies, reads and barriers still run, so
    // every wave keeps the block's pace).  act_tm: this wave's live row blocks,
    // a scalar so the skip is a scalar branch (an MFMA ignores EXEC).
    const int live_rows = static_cast<int>(tl.row1 - tl.row0) - wm * WTM;
    const int act_tm = __builtin_amdgcn_readfirstlane(
        live_rows <= 0 ? 0 : (live_rows >= WTM ? TM : (live_rows + 31) / 32));
    auto main_loop = [&](auto partial_tag, auto nc_tag) {
        constexpr bool PARTIAL = decltype(partial_tag)::value;
        constexpr int NC = decltype(nc_tag)::value;  // this wave's copies per stage
        auto mfma_range = [&](int lo, int hi, const u32x4 (&fa)[TM], const u32x4 (&fb)[TN]) {
#pragma unroll
            for (int m = lo; m < hi; ++m)
                if (!PARTIAL || m / TN < act_tm)
                    acc[m / TN][m % TN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, fa[m / TN]), __builtin_bit_cast(bf16x8, fb[m % TN]),
                        acc[m / TN][m % TN], 0, 0, 0);
        };
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st) issue_copies(st, 0, NC);
        wait_later_stages(nc_tag);
        __builtin_amdgcn_s_barrier();
        u32x4 af[2][TM], bfr[2][TN];
        read_at(a_lane(0), b_lane(0), af[0], bfr[0]);
        // copies per k-step when a stage's copies are spread over the k-steps
        // that precede the next barrier
        constexpr int CPS = (NC + KSTEPS - 2) / (KSTEPS - 1);
        for (int it = 0; it < nk; ++it) {
            // The library is built with loops starting on 64-byte
            // boundaries; three s_nop put the loop body 12 bytes past one.
            // Measured on the Mixtral-shape layer: this layout runs the w13
            // GEMM 3 % faster than the body on the boundary, and without a
            // fixed layout the loop's position (and its time, by 3-5 %)
            // moved with unrelated code changes.
            asm volatile("s_nop 0\n s_nop 0\n s_nop 0" ::: "memory");
            const uint32_t stage = (it % STAGES) * STAGE;
            static_for<KSTEPS - 1>([&](auto sc) {
                constexpr int s = decltype(sc)::value;
                read_at(stage + a_lane(s + 1), stage + b_lane(s + 1), af[(s + 1) & 1], bfr[(s + 1) & 1]);
                // stage it+STAGES-1 goes to the buffer of stage it-1, free
                // since the previous barrier
                constexpr int q0 = s * CPS < NC ? s * CPS : NC;
                constexpr int q1 = (s + 1) * CPS < NC ? (s + 1) * CPS : NC;
                issue_copies(it + STAGES - 1, q0, q1);
                mfma_range(0, kMfma, af[s & 1], bfr[s & 1]);
                if constexpr (!PARTIAL) mix_sched<kMfma, kReads, q1 - q0>();
                __builtin_amdgcn_sched_barrier(0);
            });
            // the last k-step; in the last iteration the reads after the
            // barrier fetch a buffer that is never used, so the loop body has
            // no branch
            constexpr int L = (KSTEPS - 1) & 1;
            constexpr int H = kMfma / 2;
            mfma_range(0, H, af[L], bfr[L]);
            if constexpr (!PARTIAL) __builtin_amdgcn_sched_group_barrier(0x008, H, 0);
            __builtin_amdgcn_sched_barrier(0);
            // the read offsets of stage it+1 are formed before the barrier,
            // so its reads issue as soon as the barrier opens
            uint32_t na = ((it + 1) % STAGES) * STAGE + a_lane(0);
            uint32_t nb = ((it + 1) % STAGES) * STAGE + b_lane(0);
            asm volatile("" : "+v"(na), "+v"(nb));
            // this wave's reads of stage it have landed (the MFMAs above
            // consumed the last of them); its copies of stage it+1 must land
            // too, with those of stages it+2 .. it+STAGES-1 still in flight
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            wait_later_stages(nc_tag);
            __builtin_amdgcn_s_barrier();
            // the MFMAs of the second half stay behind the barrier
            __builtin_amdgcn_sched_barrier(0);
            // reads first: the compiler keeps LDS reads behind copies into LDS
            read_at(na, nb, af[L ^ 1], bfr[L ^ 1]);
            mfma_range(H, kMfma, af[L], bfr[L]);
            if constexpr (!PARTIAL) mix_sched<kMfma - H, kReads, 0>();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // the A and B halves of the waves of a SPLIT tile run separate loops
    auto run_loop = [&](auto partial_tag) {
        if constexpr (SPLIT) {
            if (a_wave)
                main_loop(partial_tag, std::integral_constant<int, CA>{});
            else
                main_loop(partial_tag, std::integral_constant<int, CB>{});
        } else {
            main_loop(partial_tag, std::integral_constant<int, COPIES>{});
        }
    };
    if constexpr (LOOP == kLoopAuto) {
        if (tl.row1 - tl.row0 == BM)
            run_loop(std::false_type{});
        else
            run_loop(std::true_type{});
    } else {
        run_loop(std::integral_constant<bool, LOOP == kLoopGuarded>{});
    }
    // no copy may still write LDS when the block ends
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    if (use_w) {
        if (tid < BM) row_w[tid] = my_w;
        __syncthreads();
    }
    // Accumulator value v of 32x32 block (i, j) holds row lr0 + i*32 +
    // 8*(v/4) + v%4 (lr0 = this lane's first row) and column ccol of the
    // block.  Stores address rows from this lane's first row, so the row
    // offsets are compile-time multiples of the row pitch.  Tiles with all
    // BM rows live skip the per-value row test.
    const int ccol = lane % 32;
    const int lr0 = wm * WTM + (lane / 32) * 4;
    const bool full = tl.row1 - tl.row0 == BM;
    auto row_ok = [&](auto full_tag, int dr) {
        return decltype(full_tag)::value || tl.row0 + lr0 + dr < tl.row1;
    };
    if (MODE == kModeW13 && g.c_packed) {
        // act in the packed layout: the 32 columns of a lane group are one
        // 64-byte piece of their row there too
        uint16_t* act = static_cast<uint16_t*>(g.C);
        const int64_t r0 = tl.row0 + lr0;
        auto put = [&](int dr, int64_t col, float a) {
            if (row_ok(std::false_type{}, dr)) act[act_store_index(g, r0 + dr, col)] = f32_to_bf16_bits(a);
        };
        if (g.gated) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int p = 0; p < TN / 2; ++p) {
                    const int64_t col = static_cast<int64_t>(n_tile) * (BN / 2) + (wn * (TN / 2) + p) * 32 + ccol;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int dr = i * 32 + 8 * (v / 4) + v % 4;
                        const float w = use_w ? row_w[lr0 + dr] : 1.0f;
                        put(dr, col, glu_act(g, acc[i][2 * p][v] * w, acc[i][2 * p + 1][v] * w));
                    }
                }
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t col = static_cast<int64_t>(n_tile) * BN + wn * WTN + j * 32 + ccol;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int dr = i * 32 + 8 * (v / 4) + v % 4;
                        const float w = use_w ? row_w[lr0 + dr] : 1.0f;
                        put(dr, col, silu_a(acc[i][j][v] * w, g.act_alpha));
                    }
                }
        }
    } else if (MODE == kModeW13) {
        uint16_t* act = static_cast<uint16_t*>(g.C) + static_cast<int64_t>(tl.row0 + lr0) * g.I;
        if (g.gated) {
            auto epi = [&](auto full_tag, auto w_tag) {
                constexpr bool W = decltype(w_tag)::value;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int p = 0; p < TN / 2; ++p) {
                        uint16_t* out = act + n_tile * (BN / 2) + (wn * (TN / 2) + p) * 32 + ccol;
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int dr = i * 32 + 8 * (v / 4) + v % 4;
                            if (row_ok(full_tag, dr)) {
                                float gt = acc[i][2 * p][v], up = acc[i][2 * p + 1][v];
                                if constexpr (W) {
                                    const float w = reinterpret_cast<const f32x4*>(row_w + lr0 + i * 32 + 8 * (v / 4))[0][v % 4];
                                    gt *= w;
                                    up *= w;
                                }
                                out[static_cast<int64_t>(dr) * g.I] = f32_to_bf16_bits(glu_act(g, gt, up));
                            }
                        }
                    }
            };
            if (use_w)
                epi(std::false_type{}, std::true_type{});
            else if (full)
                epi(std::true_type{}, std::false_type{});
            else
                epi(std::false_type{}, std::false_type{});
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    uint16_t* out = act + n_tile * BN + wn * WTN + j * 32 + ccol;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int dr = i * 32 + 8 * (v / 4) + v % 4;
                        if (row_ok(std::false_type{}, dr)) {
                            const float w = use_w ? row_w[lr0 + dr] : 1.0f;
                            out[static_cast<int64_t>(dr) * g.I] = f32_to_bf16_bits(silu_a(acc[i][j][v] * w, g.act_alpha));
                        }
                    }
                }
        }
    } else {
        uint16_t* y = static_cast<uint16_t*>(g.C) + kpart * g.part_stride +
                      static_cast<int64_t>(tl.row0 + lr0) * g.N + n_tile * BN + wn * WTN + ccol;
        auto epi = [&](auto full_tag) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                // the 16 rows' weights: rows 8q .. 8q+3 of the block are four
                // consecutive (16-byte aligned) floats, one LDS read each
                f32x4 wq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) wq[q] = *reinterpret_cast<const f32x4*>(row_w + lr0 + i * 32 + 8 * q);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int dr = i * 32 + 8 * (v / 4) + v % 4;
                    if (!row_ok(full_tag, dr)) continue;
                    const float w = wq[v / 4][v % 4];
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        y[static_cast<int64_t>(dr) * g.N + j * 32] = f32_to_bf16_bits(acc[i][j][v] * w);
                }
            }
        };
        if (full)
            epi(std::true_type{});
        else
            epi(std::false_type{});
    }
}

template <int BM, int BN, int WM, int WN, int ROWB, int MODE>
__global__ __launch_bounds__(WM* WN* kWave) void tile_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[TileShape<BM, BN, ROWB>::SMEM];
    // w2 may split K: the n index runs over (part, n-tile), n-tile fastest,
    // so blocks resident together share the part's A columns
    const int nparts = MODE == kModeW2 ? g.ksplit : 1;
    const TilePos tp = map_block(blockIdx.x, *g.num_tiles, g.n_tiles_n * nparts, g.tiles);
    if (!tp.ok) return;
    const int kpart = tp.n / g.n_tiles_n;
    tile_body<BM, BN, WM, WN, ROWB, MODE, kLoopAuto>(g, g.tiles[tp.m], tp.n - kpart * g.n_tiles_n, kpart,
                                                nparts, smem);
}

// The tail tile runs every MFMA (its copies, not its MFMAs, set its time,
// and the unguarded loop keeps the tuned instruction schedule; measured
// faster than skipping the empty row blocks on the Mixtral-shape layer).
#ifndef MOE_TAIL_LOOP
#define MOE_TAIL_LOOP kLoopFull
#endif

// 256 x 256 tiles with 128 x 512 tail tiles.  The copies of a tile, not its
// MFMAs, set its time, so the last m-tile of an expert with at most 128 rows
// (a ragged remainder) is computed as a 128 x 512 tile: it stages 640 rows
// per k-iteration for two n-tiles instead of 512 rows for each.  Tile order:
// a group (m-tiles of one expert, as in map_block, plus the expert's tail
// tile if it has one) sweeps pairs of n-tiles; per pair its main tiles take
// both n-tiles (m fastest), then the tail tile takes the pair, so a weight
// tile is still streamed once per group.  The positions of a group form
// whole units of (n positions of a main m-tile) / 2, and units[u] describes
// the group that owns unit u; each XCD takes a contiguous eighth of all
// positions.
//
// With ext tiles, a main m-tile may also hold 257-320 rows: it runs as a
// 320 x 256 tile (tile_body's split copies), which stages 576 rows per
// k-iteration for 320 rows of output, so an expert whose rows exceed a
// multiple of 256 by a little needs one such tile instead of a 256-row tile
// plus a tail tile.  It runs every MFMA, as the tail tile does (measured on
// the Mixtral-shape w13: the guarded loop made the layer 12 % slower, the
// full loop as fast as without ext tiles).  A main m-tile of at most 192
// rows (an expert of 129-192 rows, or such a remainder) runs as a 192 x 256
// tile: 448 rows staged per k-iteration instead of 512.
template <int MODE>
__global__ __launch_bounds__(8 * kWave) void tile_kernel_tail(GemmArgs g) {
    constexpr int SM = TileShape<256, 256, 64>::SMEM, ST = TileShape<128, 512, 64>::SMEM,
                  SX = TileShape<320, 256, 64>::SMEM;
    constexpr int S1 = SM > ST ? SM : ST;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S1 > SX ? S1 : SX];
    const int nparts = MODE == kModeW2 ? g.ksplit : 1;
    const int half = g.n_tiles_n * nparts / 2;  // positions per unit (n_tiles_n is even)
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
    if (r < 2 * d.cnt) {
        const int n = 2 * pair + r / d.cnt;
        const int kpart = n / g.n_tiles_n;
        const Tile tl = g.tiles[d.first_tile + r % d.cnt];
        if (tl.row1 - tl.row0 > 256)
            tile_body<320, 256, 2, 4, 64, MODE, kLoopFull>(g, tl, n - kpart * g.n_tiles_n, kpart, nparts, smem);
        else if (tl.row1 - tl.row0 <= 192)
            tile_body<192, 256, 2, 4, 64, MODE, kLoopAuto>(g, tl, n - kpart * g.n_tiles_n, kpart, nparts, smem);
        else
            tile_body<256, 256, 2, 4, 64, MODE, kLoopAuto>(g, tl, n - kpart * g.n_tiles_n, kpart, nparts, smem);
    } else {
        const int kpart = 2 * pair / g.n_tiles_n;
        tile_body<128, 512, 2, 4, 64, MODE, MOE_TAIL_LOOP>(g, g.tiles[d.first_tile + d.cnt],
                                                           (2 * pair - kpart * g.n_tiles_n) / 2, kpart,
                                                           nparts, smem);
    }
}

// Position t of a section of the tile order that starts at m-tile m0 and
// gives each m-tile nn positions (n index fastest within a group's sweep,
// as in map_block); groups never straddle m0.
__device__ __forceinline__ TilePos tile_at(int t, int m0, int nn, const Tile* tiles) {
    const int grp = tiles[m0 + t / nn].group;
    const int first = grp >> 8, cnt = grp & 255;
    const int w = t - (first - m0) * nn;
    return TilePos{first + w % cnt, w / cnt, true};
}

// 256 x 256 tiles of a GEMM whose reduction may be split (w2): the m-tiles
// before split[0] trailing ones run whole-K, in full rounds of 256 blocks;
// the trailing groups (the last, partial round) run as g.ksplit K parts, so
// only they pay for partial outputs and the extra tile prologues and
// epilogues.  Block order: each XCD takes a contiguous eighth of the
// whole-K positions, then a contiguous eighth of the split positions (n
// index over (part, n-tile)).  m-tiles of 257-320 rows (ext tiles, as in
// tile_kernel_tail) run the 320 x 256 body.
template <int MODE>
__global__ __launch_bounds__(8 * kWave) void tile_kernel_ksplit(GemmArgs g) {
    constexpr int SM = TileShape<256, 256, 64>::SMEM, SX = TileShape<320, 256, 64>::SMEM;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SM > SX ? SM : SX];
    const int nn = g.n_tiles_n, parts = g.ksplit;
    const int nt = *g.num_tiles, ns = g.split[0];
    const int pos_a = (nt - ns) * nn, pos_b = ns * nn * parts;
    const int per_a = (pos_a + 7) / 8, per_b = (pos_b + 7) / 8;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    if (local < per_a) {
        const int t = xcd * per_a + local;
        if (t >= pos_a) return;
        const TilePos tp = tile_at(t, 0, nn, g.tiles);
        const Tile tl = g.tiles[tp.m];
        if (tl.row1 - tl.row0 > 256)
            tile_body<320, 256, 2, 4, 64, MODE, kLoopFull>(g, tl, tp.n, 0, 1, smem);
        else
            tile_body<256, 256, 2, 4, 64, MODE, kLoopAuto>(g, tl, tp.n, 0, 1, smem);
    } else if (local < per_a + per_b) {
        const int t = xcd * per_b + (local - per_a);
        if (t >= pos_b) return;
        const TilePos tp = tile_at(t, nt - ns, nn * parts, g.tiles);
        const int kpart = tp.n / nn;
        const Tile tl = g.tiles[tp.m];
        if (tl.row1 - tl.row0 > 256)
            tile_body<320, 256, 2, 4, 64, MODE, kLoopFull>(g, tl, tp.n - kpart * nn, kpart, parts, smem);
        else
            tile_body<256, 256, 2, 4, 64, MODE, kLoopAuto>(g, tl, tp.n - kpart * nn, kpart, parts, smem);
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
    const int wave = wave_index(tid);
    const int m_tile = blockIdx.x % g.max_m_tiles;
    const int n_grp = blockIdx.x / g.max_m_tiles;
    if (m_tile >= *g.num_tiles) return;
    const Tile tl = g.tiles[m_tile];
    const int64_t eltK = static_cast<int64_t>(g.Kd) * 2;
    const BSel bw = expert_weights<MODE>(g, tl.expert, 2);
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
        b_ptr[j] = bw.base + packed_offset(b_weight_row<MODE, NPW * 16, 16>(g, bw, n_grp, j * 16 + lrow), lk, bw.rb);

    f32x4 acc[TM][NPW];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < NPW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // routing weights of the 4 rows per m-subtile this lane stores (w2, or
    // w13 with the weight on the input), loaded up front so the dependent
    // loads overlap the k-loop
    float rw[TM][4];
    const bool use_w = MODE == kModeW2 || g.weight_in;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t r = tl.row0 + i * 16 + (lane / 16) * 4 + q;
            rw[i][q] = (use_w && wave == 0 && r < tl.row1)
                           ? (MODE == kModeW2 ? row_weight(g, r) : in_weight(g, r))
                           : 1.0f;
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
                for (int j = 0; j < NPW; ++j) b[u][j] = *reinterpret_cast<const u32x4*>(b_ptr[j] + off * 16);
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
        if (g.gated) {
#pragma unroll
            for (int p = 0; p < NPW / 2; ++p) {
                const int64_t col = static_cast<int64_t>(n_grp) * (NPW / 2) * 16 + p * 16 + ccol;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t r = tl.row0 + i * 16 + crow + q;
                        if (r < tl.row1)
                            act[r * g.I + col] = f32_to_bf16_bits(
                                glu_act(g, acc[i][2 * p][q] * rw[i][q], acc[i][2 * p + 1][q] * rw[i][q]));
                    }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NPW; ++j) {
                const int64_t col = static_cast<int64_t>(n_grp) * NPW * 16 + j * 16 + ccol;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t r = tl.row0 + i * 16 + crow + q;
                        if (r < tl.row1)
                            act[r * g.I + col] = f32_to_bf16_bits(silu_a(acc[i][j][q] * rw[i][q], g.act_alpha));
                    }
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
