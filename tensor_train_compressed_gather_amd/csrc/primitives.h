// primitives.h -- wave/block scans and a 3-phase device-wide scan (gfx950, wave64).
#pragma once

#include "internal.h"

#include <type_traits>
#include <utility>

namespace ttemb {

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// A value every lane of the wave holds, moved to a scalar register.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Read-only view of device data that no kernel of the current launch writes
// (table descriptors, per-table bases set by an earlier kernel).  Through the
// constant address space, wave-uniform reads become scalar loads, which do not
// wait behind the wave's outstanding vector loads and stores.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T *kconst(const T *p)
{
    return (const __attribute__((address_space(4))) T *)p;
}

// Scheduling record of one persistent block (thread 0 only): start and end
// on the constant-rate wall clock, work done, the compute unit it ran on
// (xcc, shader engine, cu and shader-array ids) and the grid size.  Plain
// vector stores.
__device__ __forceinline__ void block_stat_write(BlockStat *slot, int64_t t0, int work, int rows)
{
    if (blockIdx.x >= (unsigned)kStatBlocks) return;
    BlockStat r;
    r.t0 = t0;
    r.t1 = wall_clock64();
    r.work = work;
    r.rows = rows;
    // __smid() = xcc << 6 | se << 4 | cu; the shader-array bit (HW_ID bit 12)
    // is appended so that CUs of the two arrays of an engine stay apart
    r.cu = (int32_t)((__smid() << 1) | __builtin_amdgcn_s_getreg(GETREG_IMMED(0, 12, HW_ID)));
    r.nb = (int32_t)gridDim.x;
    slot[blockIdx.x] = r;
}

// x / d for 0 <= x < 1024 and 1 <= d <= 16 (row slots and columns of an output
// tile against d3), through one reciprocal and one multiply instead of the
// ~40-instruction integer division: floor((x + 0.5) / d) keeps a margin of
// 0.5 / d >= 1/32 on both sides of the true quotient, far above the relative
// error (< 2^-21) of the reciprocal and the product.
__device__ __forceinline__ int small_div(int x, int d)
{
    return (int)(((float)x + 0.5f) * __builtin_amdgcn_rcpf((float)d));
}

// Inclusive scan inside one 64-lane wave.
template <class T>
__device__ __forceinline__ T wave_inclusive_scan(T x)
{
    const int lane = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        T y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    return x;
}

template <class T>
__device__ __forceinline__ T wave_sum(T x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Exclusive scan over a 256-thread block; smem holds 4 entries.
template <class T>
__device__ __forceinline__ T block_exclusive_scan(T v, T *total, T *smem)
{
    const int lane = lane_id(), w = threadIdx.x >> 6;
    T x = wave_inclusive_scan(v);
    if (lane == 63) smem[w] = x;
    __syncthreads();
    T wpre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
        T s = smem[i];
        if (i < w) wpre += s;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return wpre + x - v;
}

// 3-phase exclusive scan.  Op provides
//   int64_t count() const;                       number of elements (may read device memory)
//   uint64_t value(int64_t i) const;             element i (called twice: phases 1 and 3)
//   void emit(int64_t i, uint64_t excl, uint64_t v) const;   phase 3 output
//   void total(uint64_t tot, int64_t n) const;   called once with the grand total
// Every block owns one contiguous range, so emit() sees elements in order per block.
constexpr int kScanItems = 4;

// Position of block b in a grid of nb blocks when the blocks of one XCD
// (b % 8 under the round-robin dispatch) take consecutive positions: the
// x-th eighth of the positions goes to XCD x, so the scattered accesses that
// follow a position range stay in one L2.  Identity unless nb is a multiple of 8.
__device__ __forceinline__ int xcd_slot(int b, int nb)
{
    return (nb & 7) ? b : (b & 7) * (nb >> 3) + (b >> 3);
}

// Measured: XCD-affine scan ranges made the grouping's scans slower (their
// scattered writes gained nothing, and ranges of a device-side count smaller
// than the grid crowd onto few XCDs), so block b takes range b.
__device__ __forceinline__ int scan_range(int64_t n, int64_t *lo, int64_t *hi)
{
    const int64_t tile = (int64_t)kThreads * kScanItems;
    int64_t per = (n + gridDim.x - 1) / gridDim.x;
    per = (per + tile - 1) / tile * tile;
    const int v = blockIdx.x;
    *lo = (int64_t)v * per;
    *hi = *lo + per < n ? *lo + per : n;
    return v;
}

// Scan operators: count(), value(i) for i < count(), emit(i, exclusive, value)
// and total(sum, count); an operator may also define aux(i), data of element i
// that emit then takes as a fourth argument.  Every element's value and aux
// are loaded before any emit runs: loads behind an emit's stores would wait
// for those stores (one in-order counter for both), and a load under a
// condition is waited for before the next one is issued, so the loads are
// unconditional, from positions clamped into the block's range.
template <class Op, class = void>
struct ScanHasAux {
    static constexpr bool value = false;
};
template <class Op>
struct ScanHasAux<Op, decltype((void)std::declval<const Op &>().aux(int64_t(0)))> {
    static constexpr bool value = true;
};
struct ScanNoAux {};
template <class Op, bool A = ScanHasAux<Op>::value>
struct ScanAux {
    using type = ScanNoAux;
};
template <class Op>
struct ScanAux<Op, true> {
    using type = decltype(std::declval<const Op &>().aux(int64_t(0)));
};

template <class Op>
__global__ __launch_bounds__(kThreads) void scan_phase1(Op op, uint64_t *part)
{
    __shared__ uint64_t sm[kThreads / 64];
    const int64_t n = op.count();
    int64_t lo, hi;
    const int v = scan_range(n, &lo, &hi);
    uint64_t s = 0;
    for (int64_t base = lo; base < hi; base += (int64_t)kThreads * kScanItems) {
        uint64_t x[kScanItems];
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) {
            const int64_t i = base + (int64_t)j * kThreads + threadIdx.x;
            x[j] = op.value(i < hi ? i : hi - 1);
        }
#pragma unroll
        for (int j = 0; j < kScanItems; ++j)
            if (base + (int64_t)j * kThreads + threadIdx.x < hi) s += x[j];
    }
    s = wave_sum(s);
    if (lane_id() == 0) sm[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t = 0;
        for (int i = 0; i < kThreads / 64; ++i) t += sm[i];
        part[v] = t;
    }
}

// One block of 1024 threads scans the nparts (<= kScanBlocks) partials,
// kScanBlocks / 1024 consecutive ones per thread.
template <class Op>
__global__ __launch_bounds__(1024) void scan_phase2(Op op, uint64_t *part, int nparts)
{
    constexpr int PER = kScanBlocks / 1024;
    static_assert(PER * 1024 == kScanBlocks, "partials split evenly over the threads");
    __shared__ uint64_t sm[16];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint64_t pv[PER], v = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid * PER + j;
        pv[j] = i < nparts ? part[i] : 0;
        v += pv[j];
    }
    uint64_t x = wave_inclusive_scan(v);
    if (lane == 63) sm[w] = x;
    __syncthreads();
    uint64_t wpre = 0, tot = 0;
    for (int i = 0; i < 16; ++i) {
        if (i < w) wpre += sm[i];
        tot += sm[i];
    }
    uint64_t ex = wpre + x - v;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid * PER + j;
        if (i < nparts) part[i] = ex;
        ex += pv[j];
    }
    if (tid == 0) op.total(tot, op.count());
}

template <class Op>
__global__ __launch_bounds__(kThreads) void scan_phase3(Op op, const uint64_t *part)
{
    __shared__ uint64_t sm[kThreads / 64];
    const int64_t n = op.count();
    int64_t lo, hi;
    const int v = scan_range(n, &lo, &hi);
    constexpr bool AUX = ScanHasAux<Op>::value;
    uint64_t carry = part[v];
    for (int64_t base = lo; base < hi; base += (int64_t)kThreads * kScanItems) {
        uint64_t v[kScanItems];
        typename ScanAux<Op>::type ax[kScanItems];
        uint64_t ts = 0;
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) {
            const int64_t i = base + (int64_t)threadIdx.x * kScanItems + j, ic = i < hi ? i : hi - 1;
            v[j] = op.value(ic);
            if constexpr (AUX) ax[j] = op.aux(ic);
        }
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) {
            const int64_t i = base + (int64_t)threadIdx.x * kScanItems + j;
            v[j] = i < hi ? v[j] : 0;
            ts += v[j];
        }
        uint64_t tot;
        uint64_t ex = block_exclusive_scan(ts, &tot, sm) + carry;
#pragma unroll
        for (int j = 0; j < kScanItems; ++j) {
            int64_t i = base + (int64_t)threadIdx.x * kScanItems + j;
            if constexpr (AUX) {
                if (i < hi) op.emit(i, ex, v[j], ax[j]);
            } else {
                if (i < hi) op.emit(i, ex, v[j]);
            }
            ex += v[j];
        }
        carry += tot;
    }
}

template <class Op>
hipError_t run_scan(const Op &op, uint64_t *part, int blocks, hipStream_t s)
{
    if (blocks < 1) blocks = 1;
    if (blocks > kScanBlocks) blocks = kScanBlocks;
    hipLaunchKernelGGL(scan_phase1<Op>, dim3(blocks), dim3(kThreads), 0, s, op, part);
    hipLaunchKernelGGL(scan_phase2<Op>, dim3(1), dim3(1024), 0, s, op, part, blocks);
    hipLaunchKernelGGL(scan_phase3<Op>, dim3(blocks), dim3(kThreads), 0, s, op, part);
    return hipGetLastError();
}

// Blocks for a scan over at most n elements.
inline int scan_blocks(int64_t n)
{
    int64_t b = (n + 16 * kThreads - 1) / (16 * kThreads);
    if (b < 1) b = 1;
    if (b > kScanBlocks) b = kScanBlocks;
    return (int)b;
}

// Table of a sort key: largest t with key_base[t] <= key.
__device__ __forceinline__ int table_of_key(const TableDesc *tab, int T, uint32_t key)
{
    int lo = 0, hi = T - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (tab[mid].key_base <= key) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Segment of position k in a start array st[0..T] (st non-decreasing): the
// largest t < T with st[t] <= k.
__device__ __forceinline__ int segment_of(const int32_t *st, int T, int64_t k)
{
    int lo = 0, hi = T - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (st[mid] <= k) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

} // namespace ttemb
