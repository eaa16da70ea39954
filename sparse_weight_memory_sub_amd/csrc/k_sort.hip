// k_sort.hip -- stable LSD radix sort of one chunk's read list by slot id,
// per sequence, 8 bits per pass.
//
// The memorisation write sums, for every value row, the contributions of
// all reads of that row in the chunk and divides by their count N_read
// ("Fast-weight Product Key Memory", rainbus digest step 4; paperlayer.ai
// 3.3).  Sorting the reads by slot turns that into a segmented reduction
// whose order is fixed (reads of a row stay in (token, head, rank) order),
// so the write is bitwise reproducible and needs no float atomics.
//
// Entry e = (t*H + h)*k + j of a sequence carries key = slot id (ids outside
// [0, N) become the sentinel N, which the scatter skips) and value = e.
// Each pass: count (per-tile digit histograms), then scatter: each tile's
// workgroup derives its digit offsets from all tiles' histograms (elements
// of smaller digits anywhere, plus elements of its digit in earlier tiles)
// and places its elements by a stable rank inside the tile from wavefront
// ballots, wavefronts in order.  With SortArgs::fuse (a small sort: few
// tiles in all) only the first pass has a count launch: each scatter adds
// one per element to the next pass's histogram of the tile the element
// lands in, with integer atomics (exact in any order), and the first count
// launch zeroes those histograms.
#include "fwpkm_internal.h"

namespace fwpkm {

namespace {

__device__ __forceinline__ uint32_t load_key(const SortArgs& a, int b, int pos) {
    if (a.first) {
        const int32_t s = a.idx[static_cast<size_t>(b) * a.idx_bstride + pos];
        return (s < 0 || static_cast<uint32_t>(s) >= a.N) ? a.N : static_cast<uint32_t>(s);
    }
    return a.kin[static_cast<size_t>(b) * a.M + pos];
}

template <int ITEMS>
__global__ __launch_bounds__(256) void k_sort_count(SortArgs a) {
    __shared__ uint32_t hist[256];
    const int tile = blockIdx.x, b = blockIdx.y;
    hist[threadIdx.x] = 0u;
    __syncthreads();
    const int base = tile * 256 * ITEMS;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int pos = base + it * 256 + threadIdx.x;
        if (pos < a.M) atomicAdd(&hist[(load_key(a, b, pos) >> a.shift) & 255u], 1u);
    }
    __syncthreads();
    const size_t row = (static_cast<size_t>(b) * a.tiles + tile) * 256 + threadIdx.x;
    a.counts[row] = hist[threadIdx.x];
    // the later passes' counts start from zero: their scatters add to them
    if (a.fuse)
        for (int p = 1; p < a.passes; ++p) a.counts[static_cast<size_t>(p) * a.pass_stride + row] = 0u;
}

template <int ITEMS>
__global__ __launch_bounds__(256) void k_sort_scatter(SortArgs a) {
    __shared__ uint32_t cnt[4][256];
    __shared__ uint32_t toff[256];
    __shared__ uint32_t wsum[4];
    const int tile = blockIdx.x, b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int w = 0; w < 4; ++w) cnt[w][threadIdx.x] = 0u;
    {
        // digit d = threadIdx.x: its total over all tiles and over the tiles
        // before this one, then the exclusive prefix of the totals over digits
        const uint32_t* col = a.counts + static_cast<size_t>(b) * a.tiles * 256 + threadIdx.x;
        uint32_t tot = 0u, before = 0u;
        int t = 0;
        // 32 tiles' counts requested at once (a sequence of 2^16 reads has 32
        // tiles), then 8 at a time
        for (; t + 32 <= a.tiles; t += 32) {
            uint32_t c[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) c[u] = col[static_cast<size_t>(t + u) * 256];
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                tot += c[u];
                before += (t + u < tile) ? c[u] : 0u;
            }
        }
        for (; t + 8 <= a.tiles; t += 8) {
            uint32_t c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) c[u] = col[static_cast<size_t>(t + u) * 256];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                tot += c[u];
                before += (t + u < tile) ? c[u] : 0u;
            }
        }
        for (; t < a.tiles; ++t) {
            const uint32_t c = col[static_cast<size_t>(t) * 256];
            tot += c;
            before += (t < tile) ? c : 0u;
        }
        const uint32_t incl = wave_incl_scan_u32(tot);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        uint32_t off = 0u;
        for (int w = 0; w < wave; ++w) off += wsum[w];
        toff[threadIdx.x] = off + incl - tot + before;
    }
    __syncthreads();

    constexpr int kPerWave = 64 * ITEMS;
    const int wbase = tile * 256 * ITEMS + wave * kPerWave;
    const uint64_t lt = lanemask_lt();
    uint32_t key[ITEMS], val[ITEMS], loc[ITEMS];
    // every round's key and value requested before the first ranking (the
    // ranking's LDS fences would otherwise hold each load behind the last)
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int pos = wbase + r * 64 + lane;
        const bool valid = pos < a.M;
        key[r] = valid ? load_key(a, b, pos) : 0u;
        val[r] = valid ? (a.first ? static_cast<uint32_t>(pos) : a.vin[static_cast<size_t>(b) * a.M + pos]) : 0u;
    }
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int pos = wbase + r * 64 + lane;
        const bool valid = pos < a.M;
        const uint32_t d = (key[r] >> a.shift) & 255u;
        uint64_t peers = ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (d >> bit) & 1u;
            const uint64_t bb = ballot(valid && on);
            peers &= on ? bb : ~bb;
        }
        const uint32_t rank = __popcll(peers & lt);
        const uint32_t before = valid ? cnt[wave][d] : 0u;
        wave_sync();
        if (valid && rank == 0) cnt[wave][d] = before + __popcll(peers);
        wave_sync();
        loc[r] = before + rank;
    }
    __syncthreads();
    {
        const int d = threadIdx.x;
        const uint32_t c0 = cnt[0][d], c1 = cnt[1][d], c2 = cnt[2][d];
        cnt[0][d] = 0u;
        cnt[1][d] = c0;
        cnt[2][d] = c0 + c1;
        cnt[3][d] = c0 + c1 + c2;
    }
    __syncthreads();
    // with fuse, the next pass's per-tile digit counts: each element adds one
    // to (its tile after this pass, its next digit) -- integer sums, so the
    // counts are exact in any order
    const bool next = a.fuse && a.shift + 8 < 8 * a.passes;
    uint32_t* cnext = a.counts + a.pass_stride + static_cast<size_t>(b) * a.tiles * 256;  // a.counts: this pass's
#pragma unroll
    for (int r = 0; r < ITEMS; ++r) {
        const int pos = wbase + r * 64 + lane;
        if (pos < a.M) {
            const uint32_t d = (key[r] >> a.shift) & 255u;
            const uint32_t g = toff[d] + cnt[wave][d] + loc[r];
            a.kout[static_cast<size_t>(b) * a.M + g] = key[r];
            a.vout[static_cast<size_t>(b) * a.M + g] = val[r];
            if (next) atomicAdd(&cnext[(g / (256 * ITEMS)) * 256 + ((key[r] >> (a.shift + 8)) & 255u)], 1u);
        }
    }
}

}  // namespace

hipError_t launch_sort_pass(const SortArgs& a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.tiles), static_cast<unsigned>(a.B));
    // with fuse, the scatter of the pass before has counted this pass's digits
    SortArgs c = a;
    const bool count = a.first || !a.fuse;
    if (a.fuse) c.counts = a.counts + static_cast<size_t>(a.shift / 8) * a.pass_stride;
    if (a.items == kSortItemsSmall) {
        if (count) hipLaunchKernelGGL(k_sort_count<kSortItemsSmall>, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(k_sort_scatter<kSortItemsSmall>, grid, dim3(256), 0, s, c);
    } else if (a.items == kSortItems) {
        if (count) hipLaunchKernelGGL(k_sort_count<kSortItems>, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(k_sort_scatter<kSortItems>, grid, dim3(256), 0, s, c);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fwpkm
