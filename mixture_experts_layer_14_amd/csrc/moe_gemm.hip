// moe_gemm.hip -- the two grouped expert GEMMs of the fused MoE forward on
// CDNA4 matrix cores, plus the tile schedule and the weighted combine.
//
// Operation (vLLM docs page "vllm.model_executor.layers.fused_moe.layer",
// FusedMoE: w13 [E, 2I, H] holds w1 (gate) rows then w3 (up) rows per
// _load_w13, w2 [E, H, I] is down_proj, activation "silu" with
// is_act_and_mul; SGLang page "srt/models/deepseek_v2.py", DeepseekV2MLP:
// gate_up_proj -> SiluAndMul -> down_proj):
//   w13:  act[r, n] = silu(x_t . w13[e, n, :]) * (x_t . w13[e, I + n, :])
//         for row r of expert e's segment, t = token of sorted_slots[r];
//   w2:   y[r, h]   = w_r * (act[r, :] . w2[e, h, :]),  w_r = routing weight;
//   combine: out[t, h] = sum_k y[row(t, k), h]  (+ shared expert row).
//
// Both GEMMs are "NT": A rows and B rows are contiguous along the reduction
// dimension, which is what the MFMA operand layout wants (each lane holds a
// 16-byte run of one row).  The w13 tiles load gate rows and up rows in
// interleaved blocks, so the MFMA tile holding gate columns and the one
// holding the matching up columns sit in the same lanes and SiLU-and-mul
// happens in registers.  Kernels: tile_kernel / tile_kernel_tail /
// tile_kernel_ksplit (bf16 prefill, moe_gemm_kernels.h), stream_kernel
// (bf16 decode, same file), tile_kernel_fp8 (moe_gemm_fp8.h) and, below,
// grouped_gemm_kernel for fp32 layers: BM x BN tiles of 16x16 MFMAs with
// 128 bytes of each A and B row per k-iteration in LDS (rows padded to 144
// bytes), double-buffered through registers.
#include "moe_device.h"
#include "moe_gemm_kernels.h"
#include "moe_gemm_fp8.h"
#include "moe_internal.h"
#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// tile schedule: the m-tiles of every expert segment, built on the device
// from expert_offsets so no host synchronisation is needed.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int nshared, int32_t T,
                                                           int32_t shared_base, int BM, int gm_max,
                                                           int tail_rows, int ext_rows, Tile* __restrict__ tiles,
                                                           int32_t* __restrict__ num_tiles,
                                                           GroupUnit* __restrict__ units,
                                                           int32_t* __restrict__ num_units,
                                                           int split_nn, int32_t* __restrict__ split) {
    __shared__ int32_t wave_sums[16];
    // segment: expert g, or slice g - E of the shared expert (T rows each)
    const int g = threadIdx.x;
    int32_t r0 = 0, r1 = 0;
    if (g < E) {
        // clamp to [0, routed rows] so the table can never outgrow its buffer
        r0 = min(max(offsets[g], 0), shared_base);
        r1 = min(max(offsets[g + 1], r0), shared_base);
    } else if (g < E + nshared) {
        r0 = shared_base + (g - E) * T;
        r1 = r0 + T;
    }
    // main m-tiles of BM rows (the last one possibly ragged), unless a
    // remainder of at most ext_rows - BM rows joins the last full m-tile
    // (an ext tile of up to ext_rows rows; 0: none), or a remainder of at
    // most tail_rows rows goes to a tail tile
    const int32_t rows = r1 - r0;
    const int32_t rem = rows % BM;
    const int32_t merge = rows > BM && rem > 0 && rem <= ext_rows - BM ? 1 : 0;
    const int32_t tail = !merge && rem > 0 && rem <= tail_rows ? 1 : 0;
    const int32_t nmain = rows / BM + (rem > 0 && !tail && !merge ? 1 : 0);
    const int32_t nt = nmain + tail;
    int32_t all_tiles, all_units;
    const int32_t start = block_exclusive_sum_i32<1024>(nt, wave_sums, &all_tiles);
    const int32_t ustart = block_exclusive_sum_i32<1024>(2 * nmain + tail, wave_sums, &all_units);
    // an expert's m-tiles form groups of at most gm_max, balanced in size; a
    // group's tiles sweep the n-tiles together so they share each weight
    // tile; the tail tile joins the expert's last group
    const int32_t ngroups = nt == 0 ? 0 : (nmain == 0 ? 1 : (nmain + gm_max - 1) / gm_max);
    for (int32_t c = 0; c < ngroups; ++c) {
        const int32_t first = c * nmain / ngroups, last = (c + 1) * nmain / ngroups;
        const int32_t has_tail = c == ngroups - 1 ? tail : 0;
        const int32_t cnt = last - first;
        for (int32_t j = first; j < last + has_tail; ++j) {
            Tile t;
            t.expert = g;
            t.row0 = r0 + j * BM;
            t.row1 = j + 1 < nt ? r0 + (j + 1) * BM : r1;  // the last tile ends the segment
            t.group = (start + first) * 256 + cnt;
            tiles[start + j] = t;
        }
        if (units) {
            const GroupUnit d{start + first, cnt, has_tail, ustart + 2 * first};
            for (int32_t u = 0; u < 2 * cnt + has_tail; ++u) units[ustart + 2 * first + u] = d;
        }
    }
    if (g == 0) {
        *num_tiles = all_tiles;
        if (units) *num_units = all_units;
    }
    // Split of the K-split schedule (split_nn = n-tiles per m-tile): the
    // m-tiles run whole-K in full rounds of 256 blocks, and only the trailing
    // groups that cover the last, partial round are split along K.
    // split[0] = split m-tiles (whole groups at the end of the table),
    // split[1] = first row they own (rows below it have one K part).
    if (split_nn > 0) {
        __syncthreads();  // the tile table is written
        if (g == 0) {
            const int32_t nt = all_tiles;
            const int32_t rem = static_cast<int32_t>((static_cast<int64_t>(nt) * split_nn) % 256);
            int32_t first = nt;
            if (rem > 0) {
                first = nt - (rem + split_nn - 1) / split_nn;
                first = tiles[first].group >> 8;  // back to the start of its group
            }
            split[0] = nt - first;
            split[1] = first < nt ? tiles[first].row0 : 0x7fffffff;
        }
    }
}

// ---------------------------------------------------------------------------
// MFMA policies: how two 16-byte fragments per lane (bytes [0,64) and
// [64,128) of a 128-byte k-slab, lane group l/16 owning 16 bytes of each)
// feed the matrix core.  A and B use the same lane->k mapping, so the dot
// products are exact whatever order the hardware sums k in.
// ---------------------------------------------------------------------------

struct PolBF16 {
    static constexpr int kElt = 2;
    __device__ static __forceinline__ void mma(f32x4& acc, const u32x4 (&a)[2], const u32x4 (&b)[2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                          __builtin_bit_cast(bf16x8, b[s]), acc,
                                                          0, 0, 0);
    }
    __device__ static __forceinline__ void store(void* base, int64_t idx, float v) {
        static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
    }
    __device__ static __forceinline__ float load(const void* base, int64_t idx) {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
    }
};

struct PolF32 {
    static constexpr int kElt = 4;
    __device__ static __forceinline__ void mma(f32x4& acc, const u32x4 (&a)[2], const u32x4 (&b)[2]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const f32x4 av = __builtin_bit_cast(f32x4, a[s]);
            const f32x4 bv = __builtin_bit_cast(f32x4, b[s]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc, 0, 0, 0);
        }
    }
    __device__ static __forceinline__ void store(void* base, int64_t idx, float v) {
        static_cast<float*>(base)[idx] = v;
    }
    __device__ static __forceinline__ float load(const void* base, int64_t idx) {
        return static_cast<const float*>(base)[idx];
    }
};

template <class Pol, int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM* WN* kWave) void grouped_gemm_kernel(GemmArgs g) {
    constexpr int NT = WM * WN * kWave;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr int A_ITEMS = (BM * kChunks + NT - 1) / NT;
    constexpr int B_ITEMS = (BN * kChunks + NT - 1) / NT;
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(MODE != kModeW13 || TN % 2 == 0, "w13 wave tile holds gate/up pairs");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][(BM + BN) * kLdsStride];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_index(tid);
    const int wm = wave / WN, wn = wave % WN;

    // block -> (m-tile, n-tile); m-tiles of one n-tile are adjacent so the
    // blocks sharing a weight tile run close together in time
    const int m_tile = blockIdx.x % g.max_m_tiles;
    const int n_tile = blockIdx.x / g.max_m_tiles;
    if (m_tile >= *g.num_tiles) return;
    const Tile tl = g.tiles[m_tile];
    const int64_t eltK = static_cast<int64_t>(g.Kd) * Pol::kElt;  // bytes per row
    const BSel bw = expert_weights<MODE>(g, tl.expert, Pol::kElt);

    // fixed global row addresses of this thread's load chunks
    const uint8_t* a_ptr[A_ITEMS];
    const uint8_t* b_ptr[B_ITEMS];
    bool a_on[A_ITEMS], b_on[B_ITEMS];
#pragma unroll
    for (int q = 0; q < A_ITEMS; ++q) {
        const int c = tid + q * NT;
        a_on[q] = c < BM * kChunks;
        const int row = c / kChunks, c16 = c % kChunks;
        int64_t r = tl.row0 + row;
        if (r >= tl.row1) r = tl.row0;  // ragged tail: load a valid row, never stored
        const int64_t src = a_source_row<MODE>(g, r);
        a_ptr[q] = g.A + src * eltK + c16 * 16;
    }
#pragma unroll
    for (int q = 0; q < B_ITEMS; ++q) {
        const int c = tid + q * NT;
        b_on[q] = c < BN * kChunks;
        const int row = c / kChunks, c16 = c % kChunks;
        b_ptr[q] = bw.base + packed_offset(b_weight_row<MODE, BN, 16>(g, bw, n_tile, row), c16 * 16, bw.rb);
    }

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[A_ITEMS], rb[B_ITEMS];
#pragma unroll
    for (int q = 0; q < A_ITEMS; ++q)
        if (a_on[q]) ra[q] = *reinterpret_cast<const u32x4*>(a_ptr[q]);
#pragma unroll
    for (int q = 0; q < B_ITEMS; ++q)
        if (b_on[q]) rb[q] = *reinterpret_cast<const u32x4*>(b_ptr[q]);

    const int nk = static_cast<int>(eltK / kRowBytes);
    for (int it = 0; it < nk; ++it) {
        uint8_t* sA = smem[it & 1];
        uint8_t* sB = sA + BM * kLdsStride;
#pragma unroll
        for (int q = 0; q < A_ITEMS; ++q) {
            const int c = tid + q * NT;
            if (a_on[q]) *reinterpret_cast<u32x4*>(sA + (c / kChunks) * kLdsStride + (c % kChunks) * 16) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < B_ITEMS; ++q) {
            const int c = tid + q * NT;
            if (b_on[q]) *reinterpret_cast<u32x4*>(sB + (c / kChunks) * kLdsStride + (c % kChunks) * 16) = rb[q];
        }
        __syncthreads();
        if (it + 1 < nk) {
            const int64_t off = static_cast<int64_t>(it + 1) * kRowBytes;
#pragma unroll
            for (int q = 0; q < A_ITEMS; ++q)
                if (a_on[q]) ra[q] = *reinterpret_cast<const u32x4*>(a_ptr[q] + off);
#pragma unroll
            for (int q = 0; q < B_ITEMS; ++q)
                if (b_on[q]) rb[q] = *reinterpret_cast<const u32x4*>(b_ptr[q] + off * 16);  // packed
        }
        u32x4 af[TM][2], bf[TN][2];
        const int lrow = lane % 16, lk = (lane / 16) * 16;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                af[i][s] = *reinterpret_cast<const u32x4*>(sA + (wm * WTM + i * 16 + lrow) * kLdsStride + s * 64 + lk);
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                bf[j][s] = *reinterpret_cast<const u32x4*>(sB + (wn * WTN + j * 16 + lrow) * kLdsStride + s * 64 + lk);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) Pol::mma(acc[i][j], af[i], bf[j]);
    }

    // epilogue: lane holds rows 4*(lane/16)+q, column lane%16 of each 16x16 tile
    const int ccol = lane % 16;
    const int crow = (lane / 16) * 4;
    if (MODE == kModeW13) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = tl.row0 + wm * WTM + i * 16 + crow + q;
                if (r >= tl.row1) continue;
                const float w = g.weight_in ? in_weight(g, r) : 1.0f;
                if (g.gated) {
#pragma unroll
                    for (int p = 0; p < TN / 2; ++p) {
                        const int64_t col = static_cast<int64_t>(n_tile) * (BN / 2) + (wn * (TN / 2) + p) * 16 + ccol;
                        Pol::store(g.C, r * g.I + col, glu_act(g, acc[i][2 * p][q] * w, acc[i][2 * p + 1][q] * w));
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int64_t col = static_cast<int64_t>(n_tile) * BN + wn * WTN + j * 16 + ccol;
                        Pol::store(g.C, r * g.I + col, silu_a(acc[i][j][q] * w, g.act_alpha));
                    }
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t r = tl.row0 + wm * WTM + i * 16 + crow + q;
                if (r >= tl.row1) continue;
                const float w = row_weight(g, r);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int64_t col = static_cast<int64_t>(n_tile) * BN + wn * WTN + j * 16 + ccol;
                    Pol::store(g.C, r * g.N + col, acc[i][j][q] * w);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// combine: out[t, :] = sum_k y[row(t,k), :] (+ sum_j y[T*K + j*T + t, :]),
// fixed order
// ---------------------------------------------------------------------------

template <class Pol>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ slot_to_row,
                                                      int64_t T, int K, int H, int shared,
                                                      int64_t rows, int parts,
                                                      const int32_t* __restrict__ split,
                                                      void* __restrict__ out) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t t = idx / H;
    const int h = static_cast<int>(idx % H);
    if (t >= T) return;
    const int64_t part_stride = rows * H;
    const int64_t split_row = split ? split[1] : 0;
    float s = 0.0f;
    for (int k = 0; k < K; ++k) {
        int64_t r = slot_to_row[t * K + k];
        r = r < 0 ? 0 : (r >= rows ? rows - 1 : r);
        const int np = r >= split_row ? parts : 1;
        for (int q = 0; q < np; ++q) s += Pol::load(y, q * part_stride + r * H + h);
    }
    for (int j = 0; j < shared; ++j) {  // slices of the shared expert
        const int64_t r = T * K + j * T + t;
        const int np = r >= split_row ? parts : 1;
        for (int q = 0; q < np; ++q) s += Pol::load(y, q * part_stride + r * H + h);
    }
    Pol::store(out, t * H + h, s);
}

// bf16 combine, 8 columns per thread (16-byte loads and stores).  y holds
// `parts` partial outputs of every row (a K-split w2); the sum runs in fp32
// in a fixed order: slot k = 0..K-1, then the shared expert's slices, each
// over parts.
__global__ __launch_bounds__(256) void combine_bf16x8_kernel(const uint16_t* __restrict__ y,
                                                             const int32_t* __restrict__ slot_to_row,
                                                             int64_t T, int K, int H, int shared,
                                                             int64_t rows, int parts,
                                                             const int32_t* __restrict__ split,
                                                             uint16_t* __restrict__ out) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int hv = H / 8;
    const int64_t t = idx / hv;
    const int h = static_cast<int>(idx % hv) * 8;
    if (t >= T) return;
    const int64_t part_stride = rows * H;
    const int64_t split_row = split ? split[1] : 0;
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = 0.0f;
    auto add_row = [&](int64_t r) {
        const int np = r >= split_row ? parts : 1;
        for (int q = 0; q < np; ++q) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(y + q * part_stride + r * H + h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s[2 * e] += __uint_as_float(v[e] << 16);
                s[2 * e + 1] += __uint_as_float(v[e] & 0xFFFF0000u);
            }
        }
    };
    for (int k = 0; k < K; ++k) {
        int64_t r = slot_to_row[t * K + k];
        add_row(r < 0 ? 0 : (r >= rows ? rows - 1 : r));
    }
    for (int j = 0; j < shared; ++j) add_row(T * K + j * T + t);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        o[e] = static_cast<uint32_t>(f32_to_bf16_bits(s[2 * e])) |
               (static_cast<uint32_t>(f32_to_bf16_bits(s[2 * e + 1])) << 16);
    *reinterpret_cast<u32x4*>(out + t * H + h) = o;
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------

namespace {

int64_t total_rows(const GroupedProblem& p) { return p.T * p.K + p.shared * p.T; }

// m-tiles of all segments (experts and shared slices): one partial tile per
// segment at most
int max_m_tiles(const GroupedProblem& p, int BM) {
    return static_cast<int>((total_rows(p) + BM - 1) / BM + p.E + p.shared);
}

// Average rows per expert that receives any: few rows -> weight streaming,
// many rows -> MFMA tiles.
int64_t rows_per_active_expert(const GroupedProblem& p) {
    const int64_t slots = p.T * p.K;
    const int64_t active = slots < p.E ? slots : p.E;
    return (slots + active - 1) / active;
}

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace


// Prefill tile configuration: block tile BM x BN on WM x WN waves, at most GM
// m-tiles of an expert per L2 group, ROWB bytes of every row per pipeline
// stage.  Measured on MI355X: 8 waves (two per SIMD) beat 4; 256 x 256 tiles
// pay off in both GEMMs once experts average 256 rows: each weight tile is
// then copied through L2 into LDS once per 256 rows instead of per 128 (the
// global->LDS copy stream, not the MFMAs, limits these kernels), and the
// MFMAs of a ragged last tile's empty row blocks are skipped.
#ifndef MOE_TILE_BM
#define MOE_TILE_BM 128
#endif
#ifndef MOE_TILE_BN
#define MOE_TILE_BN 256
#endif
#ifndef MOE_TILE_WM
#define MOE_TILE_WM 2
#endif
#ifndef MOE_TILE_WN
#define MOE_TILE_WN 4
#endif
#ifndef MOE_TILE_GM
#define MOE_TILE_GM 8
#endif
#ifndef MOE_TILE_ROWB
#define MOE_TILE_ROWB 128
#endif
#ifndef MOE_BIG_TILE_WN
#define MOE_BIG_TILE_WN 4
#endif
#ifndef MOE_BIG_TILE_ROWB
#define MOE_BIG_TILE_ROWB 64
#endif
// Remainders of at most this many rows (0: none) run as 128 x 512 tail
// tiles in the 256 x 256 schedule.
#ifndef MOE_TAIL_ROWS
#define MOE_TAIL_ROWS 128
#endif
// In that schedule a remainder of at most MOE_EXT_ROWS - 256 rows joins the
// expert's last 256-row tile as a 320 x 256 (ext) tile (0: no ext tiles),
// for reductions of at least MOE_EXT_MIN_K elements.  Measured (MI355X,
// interleaved runs): DeepSeek-V3-shape w13 with experts of exactly 320 rows
// 3.19 ms against 4.04 ms as 256-row plus 64-row tail tiles, routed 7 %
// faster in both GEMMs; Mixtral- and Qwen-shape w13 unchanged; the
// Qwen-shape w2 (K = 768, 24 k-iterations, where the tile's fixed costs
// weigh most) 2-3 % slower, hence the bound.
#ifndef MOE_EXT_ROWS
#define MOE_EXT_ROWS 320
#endif
#ifndef MOE_EXT_MIN_K
#define MOE_EXT_MIN_K 1024
#endif
#ifndef MOE_BIG_TILE_MIN_ROWS
#define MOE_BIG_TILE_MIN_ROWS 256
#endif
// k-steps each streaming wave keeps in flight, and the largest average rows
// per expert that still uses the streaming kernel.
#ifndef MOE_STREAM_U
#define MOE_STREAM_U 8
#endif
#ifndef MOE_STREAM_MAX_ROWS
#define MOE_STREAM_MAX_ROWS 64
#endif

// Split of the w2 GEMM's K across blocks (bf16 tile path): with few tiles the
// last wave of tiles would leave most of the 256 compute units idle, so the
// reduction is cut into parts whose bf16 partial outputs the combine sums.
// A function of the problem alone, so workspace sizing and launch agree.
#ifndef MOE_W2_BIG
#define MOE_W2_BIG 1
#endif
// The 256 x 256 tile (64-byte row slabs) for a GEMM with n output columns.
static bool big_tile(const GroupedProblem& p, int mode, int64_t n) {
    return (mode == kModeW13 || MOE_W2_BIG) && rows_per_active_expert(p) >= MOE_BIG_TILE_MIN_ROWS &&
           n % 256 == 0;
}

#ifndef MOE_W2_KSPLIT_MAX
#define MOE_W2_KSPLIT_MAX 4
#endif
// Split only the m-tiles of the last, partial round of blocks (1), or every
// m-tile (0).
#ifndef MOE_W2_KSPLIT_TAIL_ONLY
#define MOE_W2_KSPLIT_TAIL_ONLY 1
#endif
static int w2_ksplit(const GroupedProblem& p) {
    if (p.dtype != MOE_DTYPE_BF16 || rows_per_active_expert(p) <= MOE_STREAM_MAX_ROWS) return 1;
    if (p.H % MOE_TILE_BN != 0) return 1;
    constexpr int64_t kCUs = 256;
    const bool big = big_tile(p, kModeW2, p.H);
    const int64_t tiles = static_cast<int64_t>(max_m_tiles(p, big ? 256 : MOE_TILE_BM)) * (p.H / (big ? 256 : MOE_TILE_BN));
    const int64_t nk_all = static_cast<int64_t>(p.I) * 2 / (big ? MOE_BIG_TILE_ROWB : MOE_TILE_ROWB);
    int ks = 1;
    while (ks < MOE_W2_KSPLIT_MAX && tiles * ks < 8 * kCUs && nk_all / (ks + 1) >= 32) ++ks;
    return ks;
}

// Workspace of a grouped GEMM launch: the tile and unit counts, the tile
// table (m-tiles of at least 16 rows) and the unit table of a schedule with
// tail tiles (two units per 256-row m-tile at most).
static size_t tile_table_bytes(const GroupedProblem& p) {
    return align_up(sizeof(Tile) * static_cast<size_t>(max_m_tiles(p, 16)));
}

size_t gemm_tile_workspace_bytes(const GroupedProblem& p) {
    return align_up(256) + tile_table_bytes(p) +
           align_up(sizeof(GroupUnit) * 2 * static_cast<size_t>(max_m_tiles(p, 256)));
}

size_t w2_rows_workspace_bytes(const GroupedProblem& p) {
    const size_t elt = p.dtype == MOE_DTYPE_F32 ? 4 : 2;
    return align_up(static_cast<size_t>(w2_ksplit(p)) * total_rows(p) * p.H * elt);
}

// Tile table of BM-row m-tiles; with tail_rows > 0 (BM = 256 only) an
// expert's remainder of at most tail_rows rows becomes a tail tile and the
// unit table is written too.
static void build_tiles(const GroupedProblem& p, const int32_t* offsets, int BM, GemmArgs& g,
                        void* ws, hipStream_t stream, int tail_rows = 0, int split_nn = 0,
                        int ext_rows = 0) {
    int32_t* num_tiles = static_cast<int32_t*>(ws);
    int32_t* num_units = num_tiles + 1;
    int32_t* split = num_tiles + 2;
    Tile* tiles = reinterpret_cast<Tile*>(static_cast<uint8_t*>(ws) + 256);
    GroupUnit* units = tail_rows > 0 ? reinterpret_cast<GroupUnit*>(static_cast<uint8_t*>(ws) + 256 +
                                                                    tile_table_bytes(p))
                                     : nullptr;
    const TileTableKey key{ws, offsets, BM, tail_rows, split_nn, ext_rows};
    const TileTableKey* b = p.built;
    if (!b || b->ws != key.ws || b->offsets != key.offsets || b->bm != key.bm ||
        b->tail_rows != key.tail_rows || b->split_nn != key.split_nn || b->ext_rows != key.ext_rows) {
        build_tiles_kernel<<<1, 1024, 0, stream>>>(offsets, p.E, p.shared, static_cast<int32_t>(p.T),
                                                   static_cast<int32_t>(p.T * p.K), BM, MOE_TILE_GM,
                                                   tail_rows, ext_rows, tiles, num_tiles, units, num_units,
                                                   split_nn, split);
        if (p.built) *p.built = key;
    }
    g.split = split_nn > 0 ? split : nullptr;
    g.tiles = tiles;
    g.num_tiles = num_tiles;
    g.units = units;
    g.num_units = num_units;
    g.max_m_tiles = max_m_tiles(p, BM);
}

// generic 16x16 MFMA kernel (the fp32 layers)
template <class Pol, int BM, int BN, int WM, int WN, int MODE>
static hipError_t launch_grouped(const GroupedProblem& p, GemmArgs g, const int32_t* offsets,
                                 void* ws, hipStream_t stream) {
    if (g.a_packed || g.c_packed) return hipErrorInvalidValue;  // row-major act only
    build_tiles(p, offsets, BM, g, ws, stream);
    g.n_tiles_n = g.N / BN;
    const int64_t blocks = static_cast<int64_t>(g.max_m_tiles) * g.n_tiles_n;
    grouped_gemm_kernel<Pol, BM, BN, WM, WN, MODE><<<static_cast<unsigned>(blocks), WM * WN * kWave, 0, stream>>>(g);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int MODE>
static hipError_t launch_tile(const GroupedProblem& p, GemmArgs g, const int32_t* offsets, void* ws,
                              hipStream_t stream) {
    build_tiles(p, offsets, BM, g, ws, stream);
    g.n_tiles_n = g.N / BN;
    const int64_t total = static_cast<int64_t>(g.max_m_tiles) * g.n_tiles_n * (MODE == kModeW2 ? g.ksplit : 1);
    const int64_t blocks = 8 * ((total + 7) / 8);
    tile_kernel<BM, BN, WM, WN, (BM + BN >= 512 ? MOE_BIG_TILE_ROWB : MOE_TILE_ROWB), MODE><<<static_cast<unsigned>(blocks), WM * WN * kWave, 0, stream>>>(g);
    return hipGetLastError();
}

// 256 x 256 tiles with 128 x 512 tail tiles (n_tiles_n even: N % 512 == 0)
template <int MODE>
static hipError_t launch_tile_tail(const GroupedProblem& p, GemmArgs g, const int32_t* offsets, void* ws,
                                   hipStream_t stream) {
    build_tiles(p, offsets, 256, g, ws, stream, MOE_TAIL_ROWS, 0, g.Kd >= MOE_EXT_MIN_K ? MOE_EXT_ROWS : 0);
    g.n_tiles_n = g.N / 256;
    const int nparts = MODE == kModeW2 ? g.ksplit : 1;
    // units <= 2 per m-tile: every position of the schedule has a block
    const int64_t total = 2 * static_cast<int64_t>(g.max_m_tiles) * (g.n_tiles_n * nparts / 2);
    const int64_t blocks = 8 * ((total + 7) / 8);
    tile_kernel_tail<MODE><<<static_cast<unsigned>(blocks), 8 * kWave, 0, stream>>>(g);
    return hipGetLastError();
}

// w2 with a K split: 256 x 256 tiles whole-K in full rounds of 256 blocks,
// the trailing groups split into g.ksplit K parts (tile_kernel_ksplit)
template <int MODE>
static hipError_t launch_tile_ksplit(const GroupedProblem& p, GemmArgs& g, const int32_t* offsets, void* ws,
                                     hipStream_t stream) {
    g.n_tiles_n = g.N / 256;
    build_tiles(p, offsets, 256, g, ws, stream, 0, g.n_tiles_n, g.Kd >= MOE_EXT_MIN_K ? MOE_EXT_ROWS : 0);
    // every position of either section has a block; surplus blocks exit
    const int64_t whole = static_cast<int64_t>(g.max_m_tiles) * g.n_tiles_n;
    const int64_t parts = whole * g.ksplit;
    const int64_t blocks = 8 * ((whole + 7) / 8 + (parts + 7) / 8);
    tile_kernel_ksplit<MODE><<<static_cast<unsigned>(blocks), 8 * kWave, 0, stream>>>(g);
    return hipGetLastError();
}

// weight-streaming configuration: 16-column tiles per n-group for w13
// (gate/up pairs) and w2, and waves splitting K inside a block
#ifndef MOE_STREAM_NPW13
#define MOE_STREAM_NPW13 2
#endif
#ifndef MOE_STREAM_NPW2
#define MOE_STREAM_NPW2 2
#endif
#ifndef MOE_STREAM_WAVES
#define MOE_STREAM_WAVES 4
#endif
// A reduction at least this long is split over 8 waves per block instead
// (measured: Mixtral-shape w2, K = 14336, 188 -> 181 us; the shorter
// reductions are slower with 8).
#ifndef MOE_STREAM_LONG_K
#define MOE_STREAM_LONG_K 8192
#endif

template <int TM, int MODE>
static hipError_t launch_stream(const GroupedProblem& p, GemmArgs g, const int32_t* offsets, void* ws,
                                hipStream_t stream) {
    constexpr int NPW = MODE == kModeW13 ? MOE_STREAM_NPW13 : MOE_STREAM_NPW2;
    if (g.a_packed || g.c_packed) return hipErrorInvalidValue;  // row-major act only
    build_tiles(p, offsets, TM * 16, g, ws, stream);
    const int groups = g.N / (NPW * 16);
    const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(g.max_m_tiles) * groups);
    // (4-row-group tiles keep 4 waves: with 8 their registers spill)
    if constexpr (TM < 4) {
        if (g.Kd >= MOE_STREAM_LONG_K) {
            stream_kernel<TM, NPW, 8, MODE, MOE_STREAM_U><<<blocks, 8 * kWave, 0, stream>>>(g);
            return hipGetLastError();
        }
    }
    stream_kernel<TM, NPW, MOE_STREAM_WAVES, MODE, MOE_STREAM_U>
        <<<blocks, MOE_STREAM_WAVES * kWave, 0, stream>>>(g);
    return hipGetLastError();
}

bool act_packed_ok(const GroupedProblem& p) {
    // bf16: every GEMM past the weight-streaming sizes runs tile_body; fp8:
    // every GEMM runs an fp8 tile kernel
    return (p.dtype == MOE_DTYPE_BF16 && rows_per_active_expert(p) > MOE_STREAM_MAX_ROWS) ||
           p.dtype == MOE_DTYPE_FP8_E4M3;
}

// g is updated with the schedule's split table when the K-split schedule
// runs (the combine reads it)
template <int MODE>
static hipError_t bf16_gemm(const GroupedProblem& p, GemmArgs& g, const int32_t* offsets, void* ws,
                            hipStream_t stream) {
    const int64_t m = rows_per_active_expert(p);
    if (m <= MOE_STREAM_MAX_ROWS) {
        if (m <= 16) return launch_stream<1, MODE>(p, g, offsets, ws, stream);
        if (m <= 32) return launch_stream<2, MODE>(p, g, offsets, ws, stream);
        return launch_stream<4, MODE>(p, g, offsets, ws, stream);
    }
    const int n = g.N;
    if (big_tile(p, MODE, n)) {
        if (MODE == kModeW2 && g.ksplit > 1 && MOE_W2_KSPLIT_TAIL_ONLY && MOE_BIG_TILE_WN == 4 &&
            MOE_BIG_TILE_ROWB == 64)
            return launch_tile_ksplit<MODE>(p, g, offsets, ws, stream);
        if (MOE_TAIL_ROWS > 0 && n % 512 == 0 && MOE_BIG_TILE_WN == 4 && MOE_BIG_TILE_ROWB == 64)
            return launch_tile_tail<MODE>(p, g, offsets, ws, stream);
        return launch_tile<256, 256, 2, MOE_BIG_TILE_WN, MODE>(p, g, offsets, ws, stream);
    }
    if (n % MOE_TILE_BN == 0)
        return launch_tile<MOE_TILE_BM, MOE_TILE_BN, MOE_TILE_WM, MOE_TILE_WN, MODE>(p, g, offsets, ws, stream);
    if (n % 128 == 0) return launch_tile<128, 128, 2, 2, MODE>(p, g, offsets, ws, stream);  // 64 x 64 per wave
    return launch_tile<128, 64, 2, 1, MODE>(p, g, offsets, ws, stream);
}

template <int BM, int BN, int WM, int WN, int MODE>
static hipError_t launch_tile_fp8(const GroupedProblem& p, GemmArgs g, const int32_t* offsets,
                                  void* ws, hipStream_t stream) {
    build_tiles(p, offsets, BM, g, ws, stream);
    g.n_tiles_n = g.N / BN;
    const int64_t total = static_cast<int64_t>(g.max_m_tiles) * g.n_tiles_n;
    const int64_t blocks = 8 * ((total + 7) / 8);
    // scale loads of 4 k-blocks when the row's 128-value blocks come in
    // whole groups of 4 and the scale arrays start 16-byte aligned (every
    // group in bounds and aligned)
    const uintptr_t sc = reinterpret_cast<uintptr_t>(g.A_scale) | reinterpret_cast<uintptr_t>(g.B_scale) |
                         reinterpret_cast<uintptr_t>(g.B_shared_scale);
    if ((g.Kd / 128) % 4 == 0 && sc % 16 == 0)
        tile_kernel_fp8<BM, BN, WM, WN, MODE, 4><<<static_cast<unsigned>(blocks), WM * WN * kWave, 0, stream>>>(g);
    else
        tile_kernel_fp8<BM, BN, WM, WN, MODE, 1><<<static_cast<unsigned>(blocks), WM * WN * kWave, 0, stream>>>(g);
    return hipGetLastError();
}

// 256 x 256 fp8 tiles (tile_kernel_fp8_256) once experts average this many
// rows, when the rows' k blocks come in groups of four and the scale arrays
// are 16-byte aligned (its scale copies are the grouped ones)
#ifndef MOE_FP8_BIG
#define MOE_FP8_BIG 1
#endif
#ifndef MOE_FP8_BIG_MIN_ROWS
#define MOE_FP8_BIG_MIN_ROWS 128
#endif
// 256-row tiles; an expert's remainder of at most 128 rows runs as a
// 128-row tile inside the expert's group (tile_kernel_fp8_256 picks the body
// per tile): a 256 x 256 tile costs its copies and LDS reads whatever its
// live rows, so a short remainder is cheaper as half a tile, and in the
// group it shares the weight tiles the group streams through L2.
template <int MODE>
static hipError_t launch_tile_fp8_256(const GroupedProblem& p, GemmArgs g, const int32_t* offsets,
                                      void* ws, hipStream_t stream) {
    build_tiles(p, offsets, 256, g, ws, stream);
    g.n_tiles_n = g.N / 256;
    const int64_t total = static_cast<int64_t>(g.max_m_tiles) * g.n_tiles_n;
    tile_kernel_fp8_256<MODE><<<static_cast<unsigned>(8 * ((total + 7) / 8)), 8 * kWave, 0, stream>>>(g);
    return hipGetLastError();
}

// 256 x 256 fp8 tiles with 128 x 512 tail tiles (tile_kernel_fp8_tail; N a
// multiple of 512): the schedule of the bf16 tail kernel, an expert's
// remainder of at most 128 rows one tile per pair of n-tiles.
#ifndef MOE_FP8_TAIL
#define MOE_FP8_TAIL 1
#endif
template <int MODE>
static hipError_t launch_tile_fp8_tail(const GroupedProblem& p, GemmArgs g, const int32_t* offsets,
                                       void* ws, hipStream_t stream) {
    build_tiles(p, offsets, 256, g, ws, stream, 128);
    g.n_tiles_n = g.N / 256;
    // units <= 2 per m-tile: every position of the schedule has a block
    const int64_t total = 2 * static_cast<int64_t>(g.max_m_tiles) * (g.n_tiles_n / 2);
    tile_kernel_fp8_tail<MODE><<<static_cast<unsigned>(8 * ((total + 7) / 8)), 8 * kWave, 0, stream>>>(g);
    return hipGetLastError();
}

template <int MODE>
static hipError_t fp8_gemm(const GroupedProblem& p, GemmArgs g, const int32_t* offsets, void* ws,
                           hipStream_t stream) {
    const uintptr_t sc = reinterpret_cast<uintptr_t>(g.A_scale) | reinterpret_cast<uintptr_t>(g.B_scale) |
                         reinterpret_cast<uintptr_t>(g.B_shared_scale);
    if (MOE_FP8_BIG && (g.Kd / 128) % 4 == 0 && sc % 16 == 0 && g.N % 256 == 0 &&
        rows_per_active_expert(p) >= MOE_FP8_BIG_MIN_ROWS) {
        if (MOE_FP8_TAIL && g.N % 512 == 0) return launch_tile_fp8_tail<MODE>(p, g, offsets, ws, stream);
        return launch_tile_fp8_256<MODE>(p, g, offsets, ws, stream);
    }
    if constexpr (MODE == kModeW13) {
        return launch_tile_fp8<128, 256, 2, 4, MODE>(p, g, offsets, ws, stream);
    } else {
        if (p.H % 256 == 0) return launch_tile_fp8<128, 256, 2, 4, MODE>(p, g, offsets, ws, stream);
        return launch_tile_fp8<128, 128, 2, 4, MODE>(p, g, offsets, ws, stream);
    }
}

// Activation variants into the kernel arguments (limit 0: no clamp).
static void set_variants(const GroupedProblem& p, GemmArgs& g) {
    g.gated = p.gated;
    g.weight_in = p.weight_in;
    g.act_alpha = p.alpha;
    g.act_limit = p.limit > 0.0f ? p.limit : __builtin_huge_valf();
}

template <class Pol>
static hipError_t w13_for(const GroupedProblem& p, GemmArgs g, const int32_t* offsets, void* ws,
                          hipStream_t stream) {
    if (g.N % 128 != 0)  // non-gated, I an odd multiple of 64
        return launch_grouped<Pol, 64, 64, 2, 2, kModeW13>(p, g, offsets, ws, stream);
    if (rows_per_active_expert(p) <= 16)
        return launch_grouped<Pol, 16, 128, 1, 4, kModeW13>(p, g, offsets, ws, stream);
    return launch_grouped<Pol, 128, 128, 2, 2, kModeW13>(p, g, offsets, ws, stream);
}

template <class Pol>
static hipError_t w2_for(const GroupedProblem& p, GemmArgs g, const int32_t* offsets, void* ws,
                         hipStream_t stream) {
    if (p.H % 128 != 0) return launch_grouped<Pol, 16, 64, 1, 4, kModeW2>(p, g, offsets, ws, stream);
    if (rows_per_active_expert(p) <= 16) return launch_grouped<Pol, 16, 128, 1, 4, kModeW2>(p, g, offsets, ws, stream);
    return launch_grouped<Pol, 128, 128, 2, 2, kModeW2>(p, g, offsets, ws, stream);
}

hipError_t launch_w13(const GroupedProblem& p, const void* hidden, const float* hidden_scale,
                      const void* w13, const float* w13_scale, const void* shared_w13,
                      const float* shared_w13_scale, const int32_t* offsets,
                      const int32_t* sorted_slots, const float* topk_weights, void* act,
                      float* act_scale, void* ws, hipStream_t stream) {
    GemmArgs g{};
    set_variants(p, g);
    g.topk_weights = topk_weights;
    g.A_scale = hidden_scale;
    g.B_scale = w13_scale;
    g.B_shared_scale = shared_w13_scale;
    g.C_scale = act_scale;
    g.A = static_cast<const uint8_t*>(hidden);
    g.sorted_slots = sorted_slots;
    g.B = static_cast<const uint8_t*>(w13);
    g.B_shared = static_cast<const uint8_t*>(shared_w13);
    g.C = act;
    g.c_packed = p.act_packed ? 1 : 0;
    g.T = p.T;
    g.routed_rows = p.T * p.K;
    g.topk = p.K;
    g.Kd = p.H;
    g.N = p.gated ? 2 * p.I : p.I;
    g.I = p.I;
    g.Is = p.Is;
    g.E = p.E;
    if (p.dtype == MOE_DTYPE_BF16) return bf16_gemm<kModeW13>(p, g, offsets, ws, stream);
    if (p.dtype == MOE_DTYPE_F32) return w13_for<PolF32>(p, g, offsets, ws, stream);
    if (p.dtype == MOE_DTYPE_FP8_E4M3) return fp8_gemm<kModeW13>(p, g, offsets, ws, stream);
    return hipErrorNotSupported;
}

hipError_t launch_w2_combine(const GroupedProblem& p, const void* act, const float* act_scale,
                             const void* w2, const float* w2_scale, const void* shared_w2,
                             const float* shared_w2_scale, const int32_t* offsets,
                             const int32_t* sorted_slots, const int32_t* slot_to_row,
                             const float* topk_weights, void* out, void* ws,
                             hipStream_t stream) {
    const size_t tile_bytes = gemm_tile_workspace_bytes(p);
    void* y = static_cast<uint8_t*>(ws) + tile_bytes;
    GemmArgs g{};
    set_variants(p, g);
    g.A = static_cast<const uint8_t*>(act);
    g.sorted_slots = sorted_slots;
    g.B = static_cast<const uint8_t*>(w2);
    g.B_shared = static_cast<const uint8_t*>(shared_w2);
    g.topk_weights = topk_weights;
    g.C = y;
    g.a_packed = p.act_packed ? 1 : 0;
    g.T = p.T;
    g.routed_rows = p.T * p.K;
    g.topk = p.K;
    g.Kd = p.I;
    g.N = p.H;
    g.I = p.I;
    g.Is = p.Is;
    g.E = p.E;
    g.A_scale = act_scale;
    g.B_scale = w2_scale;
    g.B_shared_scale = shared_w2_scale;
    g.ksplit = w2_ksplit(p);
    g.part_stride = total_rows(p) * p.H;
    hipError_t err;
    if (p.dtype == MOE_DTYPE_BF16)
        err = bf16_gemm<kModeW2>(p, g, offsets, ws, stream);
    else if (p.dtype == MOE_DTYPE_F32)
        err = w2_for<PolF32>(p, g, offsets, ws, stream);
    else if (p.dtype == MOE_DTYPE_FP8_E4M3)
        err = fp8_gemm<kModeW2>(p, g, offsets, ws, stream);
    else
        return hipErrorNotSupported;
    if (err != hipSuccess) return err;
    const int64_t n = p.T * p.H;
    if (p.dtype != MOE_DTYPE_F32 && p.H % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
        const unsigned blocks = static_cast<unsigned>((n / 8 + 255) / 256);
        combine_bf16x8_kernel<<<blocks, 256, 0, stream>>>(static_cast<const uint16_t*>(y), slot_to_row, p.T, p.K,
                                                         p.H, p.shared, total_rows(p), g.ksplit, g.split,
                                                         static_cast<uint16_t*>(out));
    } else {
        const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
        if (p.dtype != MOE_DTYPE_F32)
            combine_kernel<PolBF16><<<blocks, 256, 0, stream>>>(y, slot_to_row, p.T, p.K, p.H, p.shared, total_rows(p), g.ksplit, g.split, out);
        else
            combine_kernel<PolF32><<<blocks, 256, 0, stream>>>(y, slot_to_row, p.T, p.K, p.H, p.shared, total_rows(p), g.ksplit, g.split, out);
    }
    return hipGetLastError();
}


}  // namespace moe
