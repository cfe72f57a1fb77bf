// moe_align.hip -- expert-contiguous, stable permutation of the T*K routing
// slots (the dispatch step of FusedMoE.forward_impl on the SGLang layer
// page: tokens grouped expert by expert before the expert GEMMs, combined
// back to token order afterwards).
//
// A deterministic counting sort in three launches; no atomic decides an
// order, so the result is bit-exact and independent of scheduling:
//   1. histogram: one wave per chunk of slots counts the chunk's experts in
//      LDS and writes counts[e][chunk];
//   2. scan: one block turns the expert-major count matrix into exclusive
//      prefix sums (the start of every (expert, chunk) run) and writes
//      expert_offsets;
//   3. scatter: one wave per chunk walks its slots 64 at a time, in order;
//      equal experts inside a 64-slot step are matched with one ballot per
//      bit of the expert id, so each slot learns how many earlier slots of
//      the step share its expert (stable rank), and a per-chunk cursor in
//      LDS carries the count from step to step.
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

constexpr int kAlignMaxExperts = 512;

__global__ __launch_bounds__(64) void align_hist_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                        int E, int64_t chunk, int nchunks,
                                                        int32_t* __restrict__ counts) {
    __shared__ int32_t cnt[kAlignMaxExperts];
    const int lane = threadIdx.x;
    const int c = blockIdx.x;
    for (int e = lane; e < E; e += kWave) cnt[e] = 0;
    __syncthreads();
    const int64_t begin = static_cast<int64_t>(c) * chunk;
    const int64_t end = begin + chunk < n ? begin + chunk : n;
    for (int64_t i = begin + lane; i < end; i += kWave) {
        const int e = ids[i];
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    for (int e = lane; e < E; e += kWave) counts[static_cast<int64_t>(e) * nchunks + c] = cnt[e];
}

// Exclusive scan over the E*nchunks counts in expert-major order, in place.
// The matrix passes through LDS in segments of 16384 counts: loaded and
// stored coalesced, each thread scans a contiguous run of 16 (LDS rows padded
// by one word per 16, so the 64 lanes' runs fall in distinct banks), the
// block scans the run sums, and a carry links the segments.
constexpr int kScanSeg = 16384, kScanRun = 16;
__device__ __forceinline__ int scan_slot(int i) { return i + i / kScanRun; }

__global__ __launch_bounds__(1024) void align_scan_kernel(int32_t* __restrict__ counts, int E,
                                                          int nchunks,
                                                          int32_t* __restrict__ offsets) {
    __shared__ int32_t buf[kScanSeg + kScanSeg / kScanRun];
    __shared__ int32_t wave_sums[16];
    const int tid = threadIdx.x;
    const int64_t m = static_cast<int64_t>(E) * nchunks;
    int32_t carry = 0;
    for (int64_t base = 0; base < m; base += kScanSeg) {
        const int n = static_cast<int>(m - base < kScanSeg ? m - base : kScanSeg);
        for (int i = tid; i < n; i += 1024) buf[scan_slot(i)] = counts[base + i];
        __syncthreads();
        const int b = tid * kScanRun, e = b + kScanRun < n ? b + kScanRun : n;
        int32_t s = 0;
        for (int i = b; i < e; ++i) s += buf[scan_slot(i)];
        int32_t seg_total;
        int32_t run = carry + block_exclusive_sum_i32<1024>(s, wave_sums, &seg_total);
        for (int i = b; i < e; ++i) {
            const int32_t c = buf[scan_slot(i)];
            buf[scan_slot(i)] = run;
            if ((base + i) % nchunks == 0) offsets[(base + i) / nchunks] = run;
            run += c;
        }
        __syncthreads();
        for (int i = tid; i < n; i += 1024) counts[base + i] = buf[scan_slot(i)];
        carry += seg_total;
        __syncthreads();
    }
    if (tid == 0) offsets[E] = carry;
}

__global__ __launch_bounds__(64) void align_scatter_kernel(const int32_t* __restrict__ ids,
                                                           int64_t n, int E, int64_t chunk,
                                                           int nchunks,
                                                           const int32_t* __restrict__ starts,
                                                           int32_t* __restrict__ sorted_slots,
                                                           int32_t* __restrict__ slot_to_row) {
    __shared__ int32_t cursor[kAlignMaxExperts];
    const int lane = threadIdx.x;
    const int c = blockIdx.x;
    for (int e = lane; e < E; e += kWave) cursor[e] = starts[static_cast<int64_t>(e) * nchunks + c];
    __syncthreads();
    const int64_t begin = static_cast<int64_t>(c) * chunk;
    const int64_t end = begin + chunk < n ? begin + chunk : n;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int64_t base = begin; base < end; base += kWave) {
        const int64_t i = base + lane;
        int e = i < end ? ids[i] : -1;
        const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
        if (!valid) e = kAlignMaxExperts;  // matches only other invalid lanes
        uint64_t same = __ballot(valid) ;
        same = valid ? same : ~same;
#pragma unroll
        for (int bit = 0; bit < 10; ++bit) {
            const bool on = (e >> bit) & 1;
            const uint64_t bal = __ballot(on);
            same &= on ? bal : ~bal;
        }
        const int before = __popcll(same & lt_mask);
        const int total = __popcll(same);
        int32_t row = 0;
        if (valid) row = cursor[e] + before;
        __syncthreads();
        if (valid) {
            sorted_slots[row] = static_cast<int32_t>(i);
            slot_to_row[i] = row;
            if (before == total - 1) cursor[e] = row + 1;
        }
        __syncthreads();
    }
}

// Whole permutation in one block for small slot counts (decode and
// Mixtral-size prefill batches):
// 16 waves each own a contiguous run of slots, loaded once into registers;
// per-wave expert counts in LDS, one scan gives the offsets and every wave's
// starting row per expert, then each wave scatters its run in slot order
// (the same stable result as the three-kernel path, in one launch instead of
// three).  Within each 64 slots, the lanes holding one expert find each
// other by ballots over the id bits; the last of them adds their number to
// the wave's count (no atomics) and, in the scatter, advances the cursor.
constexpr int kAlignSmallWaves = 16;
// Slot counts up to this run as the single block (measured: 8192 slots,
// Mixtral-shape prefill, one launch instead of three saves ~8 us; at 65536
// slots one block is slower than the three-kernel path)
#ifndef MOE_ALIGN_SMALL_MAX
#define MOE_ALIGN_SMALL_MAX 16384
#endif
constexpr int64_t kAlignSmallMax = MOE_ALIGN_SMALL_MAX;
// ids per lane when a wave's run is held in registers
constexpr int kAlignSmallPerLane =
    static_cast<int>((kAlignSmallMax + kAlignSmallWaves * kWave - 1) / (kAlignSmallWaves * kWave));

__global__ __launch_bounds__(kAlignSmallWaves * kWave) void align_small_kernel(
    const int32_t* __restrict__ ids, int64_t n, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_to_row) {
    __shared__ int32_t cnt[kAlignSmallWaves][kAlignMaxExperts];  // counts, then cursors
    __shared__ int32_t wave_sums[kAlignSmallWaves];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = wave_index(tid);
    const int chunk = static_cast<int>((n + kAlignSmallWaves - 1) / kAlignSmallWaves);
    const int begin = w * chunk;
    const int end = begin + chunk < n ? begin + chunk : static_cast<int>(n);
    // the wave's ids, slot begin + 64 j + lane in my[j] (-1 past the run)
    int32_t my[kAlignSmallPerLane];
#pragma unroll
    for (int j = 0; j < kAlignSmallPerLane; ++j) {
        const int i = begin + j * kWave + lane;
        my[j] = i < end ? ids[i] : -1;
    }
    // lanes of the same 64 holding the same expert (or, for lanes whose id
    // is out of range, the other such lanes); bits above E-1 are all zero
    const int nbits = E > 1 ? 32 - __builtin_clz(static_cast<unsigned>(E - 1)) : 0;
    auto same_expert = [&](int e, bool valid) {
        uint64_t same = __ballot(valid);
        same = valid ? same : ~same;
        for (int bit = 0; bit < nbits; ++bit) {
            const bool on = (e >> bit) & 1;
            const uint64_t bal = __ballot(on);
            same &= on ? bal : ~bal;
        }
        return same;
    };
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    for (int e = lane; e < E; e += kWave) cnt[w][e] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kAlignSmallPerLane; ++j) {
        if (begin + j * kWave >= end) break;  // wave-uniform
        const int e = my[j];
        const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
        const uint64_t same = same_expert(e, valid);
        // the last lane of each expert's group adds the group's size; a
        // wave's LDS accesses complete in order
        if (valid && __popcll(same & ~lt_mask) == 1) cnt[w][e] += __popcll(same);
    }
    __syncthreads();
    // expert `tid`: its per-wave counts become running starts within the
    // expert; tot[tid] = its total, scanned across experts below
    int32_t run = 0;
    if (tid < E) {
        for (int v = 0; v < kAlignSmallWaves; ++v) {
            const int32_t c = cnt[v][tid];
            cnt[v][tid] = run;
            run += c;
        }
    }
    int32_t total;
    const int32_t base = block_exclusive_sum_i32<kAlignSmallWaves * kWave>(tid < E ? run : 0, wave_sums, &total);
    if (tid < E) {
        offsets[tid] = base;
        for (int v = 0; v < kAlignSmallWaves; ++v) cnt[v][tid] += base;
    }
    if (tid == 0) offsets[E] = total;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kAlignSmallPerLane; ++j) {
        if (begin + j * kWave >= end) break;  // wave-uniform
        const int i = begin + j * kWave + lane;
        const int e = my[j];
        const bool valid = static_cast<unsigned>(e) < static_cast<unsigned>(E);
        const uint64_t same = same_expert(e, valid);
        const int before = __popcll(same & lt_mask);
        const int total = __popcll(same);
        int32_t row = 0;
        if (valid) row = cnt[w][e] + before;
        // this wave's cursor row is private: a wave's LDS accesses complete in
        // order, so the read above precedes the update below
        if (valid) {
            sorted_slots[row] = i;
            slot_to_row[i] = row;
            if (before == total - 1) cnt[w][e] = row + 1;
        }
    }
}

int64_t align_chunk(int64_t n) {
    // one wave per chunk, at most 256 chunks (keeps the scan matrix small)
    int64_t chunk = 1024;
    while ((n + chunk - 1) / chunk > 256) chunk *= 2;
    return chunk;
}

size_t align_workspace_bytes(int64_t n, int E) {
    const int64_t chunk = align_chunk(n);
    const int64_t nchunks = n > 0 ? (n + chunk - 1) / chunk : 1;
    return static_cast<size_t>(nchunks) * E * sizeof(int32_t);
}

hipError_t launch_align(const int32_t* ids, int64_t n, int E, int32_t* offsets,
                        int32_t* sorted_slots, int32_t* slot_to_row, void* ws, hipStream_t stream) {
    if (n <= kAlignSmallMax && E <= kAlignMaxExperts) {
        align_small_kernel<<<1, kAlignSmallWaves * kWave, 0, stream>>>(ids, n, E, offsets, sorted_slots,
                                                                        slot_to_row);
        return hipGetLastError();
    }
    const int64_t chunk = align_chunk(n);
    const int nchunks = static_cast<int>((n + chunk - 1) / chunk);
    int32_t* counts = static_cast<int32_t*>(ws);
    align_hist_kernel<<<nchunks, kWave, 0, stream>>>(ids, n, E, chunk, nchunks, counts);
    align_scan_kernel<<<1, 1024, 0, stream>>>(counts, E, nchunks, offsets);
    align_scatter_kernel<<<nchunks, kWave, 0, stream>>>(ids, n, E, chunk, nchunks, counts,
                                                        sorted_slots, slot_to_row);
    return hipGetLastError();
}

}  // namespace moe
