// moe_router.hip -- router gate logits, logits[T, E] = hidden[T, H] W_g[E, H]^T
// in fp32 (SGLang page "srt/models/deepseek_v2.py", class MoEGate: the gate
// weight is [n_routed_experts, hidden_size] in the model dtype or in fp32;
// forward returns F.linear(hidden.float(), weight) for an fp32 gate and a
// bf16 GEMM with fp32 output for a bf16 gate).
//
// bf16 hidden: MFMA 32x32x16 bf16 tiles of 64 tokens x 64 experts (128 x 128
// for many tokens), fp32 accumulation.  An fp32 gate is split on the fly into bf16 hi + lo parts
// (hi = bf16(w), lo = bf16(w - hi), |w - hi - lo| <= 2^-16 |w|), two MFMAs per
// step; each bf16 x bf16 product is exact in fp32, so the result keeps fp32
// accuracy at bf16 MFMA rate.  Few tiles (decode) split H into parts whose
// fp32 partial logits a second kernel sums in a fixed order: the reduce
// kernel (moe_router_gemm) or the top-k kernel itself (moe_router_topk).
// For few tokens the router kernel can run the top-k itself: the last blocks
// to finish their partial logits take the tokens' top-k in slices, so gate
// GEMM and top-k are one launch.
// fp32 hidden: one thread per logit, fp32 FMAs in order over H.
#include <atomic>

#include "moe_device.h"
#include "moe_internal.h"
#include "moe_topk.h"

namespace moe {
namespace {

constexpr int kRK = 64;  // k per step (one 128-byte bf16 row slab)

// Arrival counts of the router kernel's blocks at the fused top-k, one per
// launch in flight (zero when none runs on it: the last arrival wraps it
// back).  Each device holds its own array; the host hands successive
// launches successive slots, so up to kArrivalSlots launches may overlap
// on one device.
constexpr int kArrivalSlots = 64;
__device__ uint32_t router_arrivals[kArrivalSlots];

// Blocks that run the fused top-k: one token per wave, at most 64 blocks
// (the blocks waiting for the others' partial logits).
__host__ __device__ inline uint32_t fused_topk_blocks(int64_t T, int64_t total, int waves) {
    int64_t f = (T + waves - 1) / waves;
    f = f < 64 ? f : 64;
    return static_cast<uint32_t>(f < total ? f : total);
}

// 16-byte slot s of LDS row r (128-byte rows): XOR swizzle so the 32 rows one
// MFMA operand read touches spread over all banks
__device__ __forceinline__ int rslot(int r, int s) { return s ^ (r & 7); }

// Tile of BM tokens x BN experts on WM x WN waves (each wave (BM/WM) x
// (BN/WN), 32 x 32 MFMA blocks); 64 x 64 on 4 waves for few tokens, 128 x
// 128 on 8 waves for many (half the hidden and gate re-reads per logit, and
// two independent MFMA chains per wave).  FUSE_VPL > 0: the kernel also
// runs the top-k (tk; experts per lane FUSE_VPL) on `out` once all of it is
// written.
template <bool GATE_F32, int BM, int BN, int WM, int WN, int FUSE_VPL = 0>
__global__ __launch_bounds__(WM* WN* kWave) void router_gemm_kernel(
    const uint16_t* __restrict__ x, const void* __restrict__ gate, int64_t T, int E, int H,
    int parts, float* __restrict__ out, TopkArgs tk, int slot = 0) {
    constexpr int NT = WM * WN * kWave;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
    constexpr int NB = GATE_F32 ? 2 : 1;  // gate planes in LDS: hi (and lo)
    constexpr int STAGE = (BM + NB * BN) * kRK * 2;
    constexpr int A_LD = BM * 8 / NT;                        // 16-byte A loads per thread
    constexpr int B_LD = BN * (GATE_F32 ? 16 : 8) / NT;      // 16-byte gate loads per thread
    static_assert(BM * 8 % NT == 0 && BN * (GATE_F32 ? 16 : 8) % NT == 0, "loads split evenly");
    static_assert(TM >= 1 && TN >= 1, "wave tile of whole 32 x 32 blocks");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_index(tid);
    const int wm = wave / WN, wn = wave % WN;
    // block -> (token tile, expert tile): block b runs on XCD b % 8; each XCD
    // takes a contiguous eighth of the tiles in token-major order, so the
    // expert tiles of one token tile run together on one XCD and read its
    // hidden rows from that XCD's L2 (token-tile-fastest order re-read every
    // hidden row once per expert tile)
    const int tiles_e = (E + BN - 1) / BN;
    const int64_t tiles = ((T + BM - 1) / BM) * tiles_e;
    const int64_t per = (tiles + 7) / 8;
    const int64_t pos = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((blockIdx.x >> 3) >= per || pos >= tiles) return;
    const int64_t t0 = pos / tiles_e * BM;
    const int e0 = static_cast<int>(pos % tiles_e) * BN;
    const int part = blockIdx.z;
    const int nk_all = H / kRK;
    const int k_first = part * nk_all / parts;
    const int nk = (part + 1) * nk_all / parts - k_first;

    // loads of one k-step into registers: A (bf16) 8 chunks of 16 bytes per
    // row, the gate 8 (bf16) or 16 (fp32) per row; rows past T or E repeat
    // the last row (computed, never stored)
    u32x4 ra[A_LD], rb[B_LD];
    auto load = [&](int kit) {
        const int64_t k0 = static_cast<int64_t>(k_first + kit) * kRK;
#pragma unroll
        for (int j = 0; j < A_LD; ++j) {
            const int idx = tid + j * NT;
            const int r = idx >> 3, s = idx & 7;
            const int64_t t = t0 + r < T ? t0 + r : T - 1;
            ra[j] = *reinterpret_cast<const u32x4*>(x + t * H + k0 + s * 8);
        }
        if constexpr (!GATE_F32) {
            const uint16_t* g = static_cast<const uint16_t*>(gate);
#pragma unroll
            for (int j = 0; j < B_LD; ++j) {
                const int idx = tid + j * NT;
                const int r = idx >> 3, s = idx & 7;
                const int64_t e = e0 + r < E ? e0 + r : E - 1;
                rb[j] = *reinterpret_cast<const u32x4*>(g + e * H + k0 + s * 8);
            }
        } else {
            const float* g = static_cast<const float*>(gate);
#pragma unroll
            for (int j = 0; j < B_LD; ++j) {
                const int idx = tid + j * NT;  // 4 floats each: 16 per row
                const int r = idx >> 4, c = (idx & 15) * 4;
                const int64_t e = e0 + r < E ? e0 + r : E - 1;
                rb[j] = *reinterpret_cast<const u32x4*>(g + e * H + k0 + c);
            }
        }
    };
    auto store = [&](int buf) {
        uint8_t* sA = smem + buf * STAGE;
        uint8_t* sB = sA + BM * kRK * 2;
#pragma unroll
        for (int j = 0; j < A_LD; ++j) {
            const int idx = tid + j * NT;
            const int r = idx >> 3, s = idx & 7;
            *reinterpret_cast<u32x4*>(sA + r * 128 + rslot(r, s) * 16) = ra[j];
        }
        if constexpr (!GATE_F32) {
#pragma unroll
            for (int j = 0; j < B_LD; ++j) {
                const int idx = tid + j * NT;
                const int r = idx >> 3, s = idx & 7;
                *reinterpret_cast<u32x4*>(sB + r * 128 + rslot(r, s) * 16) = rb[j];
            }
        } else {
            uint8_t* sL = sB + BN * kRK * 2;
#pragma unroll
            for (int j = 0; j < B_LD; ++j) {
                const int idx = tid + j * NT;
                const int r = idx >> 4, c = (idx & 15) * 4;
                uint32_t hi[2], lo[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const float w0 = __uint_as_float(rb[j][2 * q]), w1 = __uint_as_float(rb[j][2 * q + 1]);
                    const uint16_t h0 = f32_to_bf16_bits(w0), h1 = f32_to_bf16_bits(w1);
                    const uint16_t l0 = f32_to_bf16_bits(w0 - bf16_bits_to_f32(h0));
                    const uint16_t l1 = f32_to_bf16_bits(w1 - bf16_bits_to_f32(h1));
                    hi[q] = h0 | (static_cast<uint32_t>(h1) << 16);
                    lo[q] = l0 | (static_cast<uint32_t>(l1) << 16);
                }
                // 4 values = 8 bytes: half of 16-byte slot c / 8
                const int off = r * 128 + rslot(r, c >> 3) * 16 + (c & 7) * 2;
                *reinterpret_cast<uint2*>(sB + off) = make_uint2(hi[0], hi[1]);
                *reinterpret_cast<uint2*>(sL + off) = make_uint2(lo[0], lo[1]);
            }
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    const int kh = lane >> 5;

    load(0);
    store(0);
    __syncthreads();
    for (int kit = 0; kit < nk; ++kit) {
        const int buf = kit & 1;
        if (kit + 1 < nk) load(kit + 1);
        const uint8_t* sA = smem + buf * STAGE;
        const uint8_t* sB = sA + BM * kRK * 2;
#pragma unroll
        for (int ks = 0; ks < kRK / 16; ++ks) {
            const int s = ks * 2 + kh;
            u32x4 a[TM], b[TN], bl[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int ar = wm * (BM / WM) + i * 32 + (lane & 31);
                a[i] = *reinterpret_cast<const u32x4*>(sA + ar * 128 + rslot(ar, s) * 16);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int br = wn * (BN / WN) + j * 32 + (lane & 31);
                b[j] = *reinterpret_cast<const u32x4*>(sB + br * 128 + rslot(br, s) * 16);
                if constexpr (GATE_F32)
                    bl[j] = *reinterpret_cast<const u32x4*>(sB + BN * kRK * 2 + br * 128 + rslot(br, s) * 16);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
                    if constexpr (GATE_F32)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, bl[j]), acc[i][j], 0, 0,
                            0);
                }
        }
        __syncthreads();  // every wave is done with `buf` and with the other buffer
        if (kit + 1 < nk) {
            store(buf ^ 1);
            __syncthreads();
        }
    }

    // acc[i][j][v] holds token row i*32 + 8*(v/4) + 4*(lane/32) + v%4 and
    // expert column j*32 + lane%32 of the wave tile
    float* o = out + static_cast<int64_t>(part) * T * E;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int e = e0 + wn * (BN / WN) + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t t = t0 + wm * (BM / WM) + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
                if (t < T && e < E) {
                    if constexpr (FUSE_VPL > 0)  // written through to memory: read by other blocks below
                        __hip_atomic_store(reinterpret_cast<uint32_t*>(o + t * E + e), __float_as_uint(acc[i][j][v]),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else
                        o[t * E + e] = acc[i][j][v];
                }
            }
        }

    if constexpr (FUSE_VPL > 0) {
        // Every block counts its arrival once its partial logits are out; the
        // last `fin` to arrive wait for the count to wrap (all arrived), then
        // run the top-k of tokens slot*NW + wave, slot*NW + wave + fin*NW, ...
        // No block waits before it arrives, and at most `fin` (<= 64) wait, so
        // the blocks not yet arrived are running or find a free slot: the wait
        // ends.  Its bound only keeps a wait finite.
        // The partial logits went out as device-coherent stores: once they are
        // complete, the arrival count may move (no write-back of the whole L2,
        // as a release fence would do).
        __shared__ uint32_t s_ticket;
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const uint32_t total = static_cast<uint32_t>(tiles * parts);
        uint32_t* const arrivals = router_arrivals + slot;
        if (tid == 0) s_ticket = atomicInc(arrivals, total - 1);  // the last arrival wraps to 0
        __syncthreads();
        const uint32_t ticket = s_ticket;
        const uint32_t fin = fused_topk_blocks(T, total, WM * WN);
        if (ticket + fin < total) return;
        if (tid == 0 && ticket + 1 < total) {
            for (uint32_t n = 0; n < (1u << 24); ++n) {
                if (__hip_atomic_load(arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) break;
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // no stale copy of the other blocks' partial logits
        const int64_t slot = ticket - (total - fin);
        for (int64_t t = slot * (WM * WN) + wave; t < T; t += static_cast<int64_t>(fin) * (WM * WN))
            topk_row<FUSE_VPL, topk_part_batch(FUSE_VPL, 32)>(tk, t, lane);
    }
}

// 128 tokens x 128 experts on 8 waves (64 x 32 each), for many tokens: the
// hidden rows and the gate rows (bf16, or fp32 as stored) are copied global
// -> LDS by global_load_lds into a ring of 3 stages of 64 k (the copies of
// the next two steps stay in flight while one multiplies; one barrier per
// step), and an fp32 gate is split into bf16 hi + lo as its fragments are
// read (round to nearest even, as the staged split of the 64 x 64 kernel),
// so the logits are the same bits.  LDS rows: 128 bytes (bf16, 8 slots of 16
// bytes) or 256 bytes (fp32, 16 slots), slot s of row r stored at s ^ (r % 8)
// or s ^ (r % 16): the rows an operand read touches spread over all banks.
template <bool GATE_F32>
__global__ __launch_bounds__(512) void router_gemm_lds_kernel(const uint16_t* __restrict__ x,
                                                              const void* __restrict__ gate, int64_t T,
                                                              int E, int H, int parts,
                                                              float* __restrict__ out) {
    constexpr int BM = 128, BN = 128, WM = 2, WN = 4, NW = 8;
    constexpr int GROWB = GATE_F32 ? 256 : 128;          // gate bytes per row and step
    constexpr int GSLOTS = GROWB / 16;
    constexpr int A_BYTES = BM * 128, G_BYTES = BN * GROWB;
    constexpr int STAGE = A_BYTES + G_BYTES;
    constexpr int STAGES = 3;
    constexpr int A_CP = A_BYTES / 1024 / NW, G_CP = G_BYTES / 1024 / NW;  // copies per wave and step
    constexpr int CP = A_CP + G_CP;
    constexpr int TM = BM / WM / 32, TN = BN / WN / 32;  // 2 x 1
    static_assert(A_BYTES % (1024 * NW) == 0 && G_BYTES % (1024 * NW) == 0, "copies split evenly");
    static_assert(STAGES * STAGE <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_index(tid);
    const int wm = wave / WN, wn = wave % WN;
    // block -> (token tile, expert tile), XCD-aware as in router_gemm_kernel
    const int tiles_e = (E + BN - 1) / BN;
    const int64_t tiles = ((T + BM - 1) / BM) * tiles_e;
    const int64_t per = (tiles + 7) / 8;
    const int64_t pos = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((blockIdx.x >> 3) >= per || pos >= tiles) return;
    const int64_t t0 = pos / tiles_e * BM;
    const int e0 = static_cast<int>(pos % tiles_e) * BN;
    const int part = blockIdx.z;
    const int nk_all = H / kRK;
    const int k_first = part * nk_all / parts;
    const int nk = (part + 1) * nk_all / parts - k_first;

    // sources of this lane's 16-byte slot in each copy (the swizzle is an
    // involution: the lane filling slot s of row r loads chunk s ^ f(r));
    // rows past T or E repeat the last row (computed, never stored)
    const uint8_t* src[CP];
#pragma unroll
    for (int q = 0; q < A_CP; ++q) {
        const int c = wave * A_CP + q;
        const int row = c * 8 + lane / 8, chunk = (lane % 8) ^ (row % 8);
        const int64_t t = t0 + row < T ? t0 + row : T - 1;
        src[q] = reinterpret_cast<const uint8_t*>(x + t * H) + static_cast<int64_t>(k_first) * 128 + chunk * 16;
    }
#pragma unroll
    for (int q = 0; q < G_CP; ++q) {
        const int c = wave * G_CP + q;
        const int row = c * (1024 / GROWB) + lane / GSLOTS;
        const int chunk = (lane % GSLOTS) ^ (row % GSLOTS);
        const int64_t e = e0 + row < E ? e0 + row : E - 1;
        src[A_CP + q] = static_cast<const uint8_t*>(gate) + e * H * (GATE_F32 ? 4 : 2) +
                        static_cast<int64_t>(k_first) * GROWB + chunk * 16;
    }
    auto issue = [&](int kit) {
        const int kc = kit < nk ? kit : nk - 1;  // past the end: a repeat nobody reads
        uint8_t* st = smem + (kit % STAGES) * STAGE;
#pragma unroll
        for (int q = 0; q < A_CP; ++q)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src[q] + static_cast<int64_t>(kc) * 128),
                                             (__attribute__((address_space(3))) void*)(st + (wave * A_CP + q) * 1024),
                                             16, 0, 0);
#pragma unroll
        for (int q = 0; q < G_CP; ++q)
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void*>(src[A_CP + q] + static_cast<int64_t>(kc) * GROWB),
                (__attribute__((address_space(3))) void*)(st + A_BYTES + (wave * G_CP + q) * 1024), 16, 0, 0);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    const int kh = lane >> 5, lr = lane & 31;

    issue(0);
    issue(1);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (CP & 15) | ((CP >> 4) << 14));  // stage 0 landed
    __builtin_amdgcn_s_barrier();
    for (int kit = 0; kit < nk; ++kit) {
        // stage kit+2 into the buffer of stage kit-1 (read before the last barrier)
        issue(kit + 2);
        const uint8_t* sA = smem + (kit % STAGES) * STAGE;
        const uint8_t* sG = sA + A_BYTES;
#pragma unroll
        for (int ks = 0; ks < kRK / 16; ++ks) {
            const int s = ks * 2 + kh;  // bf16 chunk of this lane's 8 k values
            u32x4 a[TM], b[TN], bl[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * (BM / WM) + i * 32 + lr;
                a[i] = *reinterpret_cast<const u32x4*>(sA + r * 128 + (s ^ (r % 8)) * 16);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * (BN / WN) + j * 32 + lr;
                if constexpr (!GATE_F32) {
                    b[j] = *reinterpret_cast<const u32x4*>(sG + r * 128 + (s ^ (r % 8)) * 16);
                } else {
                    // 8 floats: chunks 2s and 2s + 1 of the 256-byte row
                    const u32x4 w0 = *reinterpret_cast<const u32x4*>(sG + r * 256 + ((2 * s) ^ (r % 16)) * 16);
                    const u32x4 w1 = *reinterpret_cast<const u32x4*>(sG + r * 256 + ((2 * s + 1) ^ (r % 16)) * 16);
                    const float f[8] = {__uint_as_float(w0[0]), __uint_as_float(w0[1]), __uint_as_float(w0[2]),
                                        __uint_as_float(w0[3]), __uint_as_float(w1[0]), __uint_as_float(w1[1]),
                                        __uint_as_float(w1[2]), __uint_as_float(w1[3])};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        bf16x2 h;
                        h[0] = static_cast<__bf16>(f[2 * q]);
                        h[1] = static_cast<__bf16>(f[2 * q + 1]);
                        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
                        bf16x2 l;
                        l[0] = static_cast<__bf16>(f[2 * q] - __uint_as_float(hb << 16));
                        l[1] = static_cast<__bf16>(f[2 * q + 1] - __uint_as_float(hb & 0xFFFF0000u));
                        b[j][q] = hb;
                        bl[j][q] = __builtin_bit_cast(uint32_t, l);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
                    if constexpr (GATE_F32)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, bl[j]), acc[i][j], 0, 0,
                            0);
                }
        }
        // this wave's reads of stage kit are done and its copies of stage
        // kit+1 landed (stage kit+2's may stay in flight); then everyone's
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_waitcnt(0x0F70 | (CP & 15) | ((CP >> 4) << 14));
        __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no copy may still write LDS

    float* o = out + static_cast<int64_t>(part) * T * E;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int e = e0 + wn * (BN / WN) + j * 32 + lr;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t t = t0 + wm * (BM / WM) + i * 32 + 8 * (v / 4) + 4 * kh + (v % 4);
                if (t < T && e < E) o[t * E + e] = acc[i][j][v];
            }
        }
}

// logits = sum of the parts' partial logits, in part order
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ partial,
                                                            int64_t n, int parts,
                                                            float* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = partial[i];
    for (int p = 1; p < parts; ++p) s += partial[p * n + i];
    out[i] = s;
}

// fp32 hidden: one thread per (token, expert), fp32 FMAs in h order
template <bool GATE_F32>
__global__ __launch_bounds__(256) void router_f32_kernel(const float* __restrict__ x,
                                                         const void* __restrict__ gate, int64_t T,
                                                         int E, int H, float* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= T * E) return;
    const int64_t t = i / E;
    const int e = static_cast<int>(i - t * E);
    float s = 0.0f;
    for (int h = 0; h < H; ++h) {
        const float w = GATE_F32 ? static_cast<const float*>(gate)[static_cast<int64_t>(e) * H + h]
                                 : bf16_bits_to_f32(static_cast<const uint16_t*>(gate)[static_cast<int64_t>(e) * H + h]);
        s = fmaf(x[t * H + h], w, s);
    }
    out[i] = s;
}

// Tile and parts of H for the MFMA path.  Many tokens take the 128 x 128
// tile; few take 64 x 64 with H split into parts (at least two k-steps each)
// so that the blocks cover the chip, their fp32 partial logits summed in
// part order by the consumer (router_reduce_kernel or the top-k kernel).
struct RouterPlan {
    bool big;
    int parts;
};

RouterPlan router_plan(int64_t T, int E, int H) {
    const int nk_all = H / kRK;
    const int64_t big_tiles = ((T + 127) / 128) * ((E + 127) / 128);
    RouterPlan pl{big_tiles >= 64, 1};
    const int64_t tiles = pl.big ? big_tiles : ((T + 63) / 64) * ((E + 63) / 64);
    const int64_t want = pl.big ? 256 : 512;
    while (pl.parts < 32 && tiles * pl.parts < want && nk_all / (pl.parts * 2) >= 2) pl.parts *= 2;
    return pl;
}

}  // namespace

int router_parts(int64_t T, int E, int H) { return router_plan(T, E, H).parts; }

size_t router_workspace_bytes(int64_t T, int E, int H, int act_dtype) {
    if (T <= 0) return 0;
    // the partial logits (bf16 hidden, split H), or one logits buffer for the
    // fused router + top-k when the caller keeps no logits
    const int parts = act_dtype == 1 /* bf16 */ ? router_parts(T, E, H) : 1;
    return static_cast<size_t>(parts) * T * E * sizeof(float);
}

hipError_t launch_router_partials(const void* hidden, int act_dtype, const void* gate,
                                  int gate_dtype, int64_t T, int E, int H, float* partials,
                                  int* parts_out, hipStream_t stream) {
    const bool gf32 = gate_dtype == 0;
    if (act_dtype != 1) {  // fp32 hidden: one pass, no parts
        const unsigned blocks = static_cast<unsigned>((T * E + 255) / 256);
        if (gf32)
            router_f32_kernel<true><<<blocks, 256, 0, stream>>>(static_cast<const float*>(hidden), gate, T, E, H, partials);
        else
            router_f32_kernel<false><<<blocks, 256, 0, stream>>>(static_cast<const float*>(hidden), gate, T, E, H, partials);
        *parts_out = 1;
        return hipGetLastError();
    }
    const RouterPlan pl = router_plan(T, E, H);
    const uint16_t* x = static_cast<const uint16_t*>(hidden);
    if (pl.big) {
        const int64_t tiles = ((T + 127) / 128) * ((E + 127) / 128);
        const dim3 grid(static_cast<unsigned>(8 * ((tiles + 7) / 8)), 1, static_cast<unsigned>(pl.parts));
        if (gf32)
            router_gemm_lds_kernel<true><<<grid, 512, 0, stream>>>(x, gate, T, E, H, pl.parts, partials);
        else
            router_gemm_lds_kernel<false><<<grid, 512, 0, stream>>>(x, gate, T, E, H, pl.parts, partials);
    } else {
        const int64_t tiles = ((T + 63) / 64) * ((E + 63) / 64);
        const dim3 grid(static_cast<unsigned>(8 * ((tiles + 7) / 8)), 1, static_cast<unsigned>(pl.parts));
        const TopkArgs none{};
        if (gf32)
            router_gemm_kernel<true, 64, 64, 2, 2><<<grid, 256, 0, stream>>>(x, gate, T, E, H, pl.parts, partials, none);
        else
            router_gemm_kernel<false, 64, 64, 2, 2><<<grid, 256, 0, stream>>>(x, gate, T, E, H, pl.parts, partials, none);
    }
    *parts_out = pl.parts;
    return hipGetLastError();
}

bool router_topk_one_launch(int64_t T, int E, int H, int act_dtype) {
    return act_dtype == 1 && T > 0 && !router_plan(T, E, H).big && T <= 256;
}

// Successive fused launches (of every instantiation) take successive
// arrival counters.
static std::atomic<uint32_t> next_arrival_slot{0};

template <int VPL>
static void launch_fused(bool gf32, dim3 grid, const uint16_t* x, const void* gate, int64_t T, int E,
                         int H, int parts, float* partials, const TopkArgs& tk, hipStream_t stream) {
    const int slot = static_cast<int>(next_arrival_slot.fetch_add(1, std::memory_order_relaxed) % kArrivalSlots);
    if (gf32)
        router_gemm_kernel<true, 64, 64, 2, 2, VPL><<<grid, 256, 0, stream>>>(x, gate, T, E, H, parts, partials, tk, slot);
    else
        router_gemm_kernel<false, 64, 64, 2, 2, VPL><<<grid, 256, 0, stream>>>(x, gate, T, E, H, parts, partials, tk, slot);
}

hipError_t launch_router_topk(const void* hidden, const void* gate, int gate_dtype, int64_t T, int E,
                              int H, float* partials, float* logits_out, const float* bias, int K,
                              int scoring, int renorm, int G, int TG, float rsf, int32_t* ids,
                              float* weights, hipStream_t stream) {
    const RouterPlan pl = router_plan(T, E, H);
    const TopkArgs tk{partials, pl.parts, T * E, logits_out, bias, T, E, K, scoring, renorm, G, TG, rsf, ids, weights};
    const int64_t tiles = ((T + 63) / 64) * ((E + 63) / 64);
    const dim3 grid(static_cast<unsigned>(8 * ((tiles + 7) / 8)), 1, static_cast<unsigned>(pl.parts));
    const uint16_t* x = static_cast<const uint16_t*>(hidden);
    const bool gf32 = gate_dtype == 0;
    const int vpl = (E + kWave - 1) / kWave;
    if (vpl <= 1)
        launch_fused<1>(gf32, grid, x, gate, T, E, H, pl.parts, partials, tk, stream);
    else if (vpl <= 2)
        launch_fused<2>(gf32, grid, x, gate, T, E, H, pl.parts, partials, tk, stream);
    else if (vpl <= 4)
        launch_fused<4>(gf32, grid, x, gate, T, E, H, pl.parts, partials, tk, stream);
    else
        launch_fused<8>(gf32, grid, x, gate, T, E, H, pl.parts, partials, tk, stream);
    return hipGetLastError();
}

hipError_t launch_router(const void* hidden, int act_dtype, const void* gate, int gate_dtype,
                         int64_t T, int E, int H, float* logits, void* ws, hipStream_t stream) {
    const int parts = act_dtype == 1 ? router_parts(T, E, H) : 1;
    float* dst = parts > 1 ? static_cast<float*>(ws) : logits;
    int got = 1;
    hipError_t err = launch_router_partials(hidden, act_dtype, gate, gate_dtype, T, E, H, dst, &got, stream);
    if (err != hipSuccess) return err;
    if (got > 1) {
        const int64_t n = T * E;
        router_reduce_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(dst, n, got, logits);
    }
    return hipGetLastError();
}

}  // namespace moe
