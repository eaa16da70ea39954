// rows_probe.hip -- rates that HBM sustains for the value rows' access
// patterns on this GPU, as ceilings for the FwPKM value-row kernels.
//
// The layer reads value rows at random (the gather) and writes each row a
// chunk's reads touched once, in slot order, as a read-modify-write (the
// "Fast-weight Product Key Memory" chunk write: the aggregated gradient of a
// row applied to that row).  Rows here are 1 KiB (512 bf16, the 2^20-slot
// layer's row).  A wavefront takes `per` consecutive entries of a row list
// and moves each row with one 16-byte access per lane, R rows at a time:
//   mode 0  read R rows, fold them into a per-lane checksum;
//   mode 1  read R rows, then write the R rows back modified;
//   mode 2  as 1, software-pipelined: the next R rows are requested before
//           the current R are written (two register sets);
//   mode 3  read R rows into LDS with direct global-to-LDS loads (one wave
//           per workgroup, R KiB of LDS each), then write them back modified
//           from LDS.
// A plain sequential copy gives the streaming rate for comparison.  Not part
// of the layer: a measurement library loaded by bench.py --ceiling.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kRow = 1024;  // bytes per row, 64 lanes x 16 B

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ u32x4 ld_nt(const unsigned char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st_nt(unsigned char* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// One 16-byte direct global-to-LDS load per lane: the wave's 64 x 16 bytes
// land contiguously at `lds`.  (Kept in a device function: the host pass
// of a kernel template does not see the target builtin.)
__device__ __forceinline__ void lds_load16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// Row r's bytes for this lane.
__device__ __forceinline__ unsigned char* lane_row(unsigned char* base, uint32_t r, int lane) {
    return base + static_cast<size_t>(r) * kRow + static_cast<size_t>(lane) * 16;
}

template <int R, int MODE>
__global__ __launch_bounds__(256) void k_rows(const uint32_t* rows, int nrows, int per, unsigned char* base,
                                              uint32_t* out) {
    const int lane = threadIdx.x & 63;
    const int wid = static_cast<int>((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
    const int first = wid * per;
    if (first >= nrows) return;
    const int cnt = min(per, nrows - first);
    // lane l holds the wave's l-th row id; rows are taken from it by readlane
    const uint32_t my = lane < cnt ? rows[first + lane] : 0u;
    auto row = [&](int j) { return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(my), j)); };
    uint32_t acc = 0;
    if constexpr (MODE == 0 || MODE == 1) {
        for (int j0 = 0; j0 < cnt; j0 += R) {
            u32x4 x[R];
#pragma unroll
            for (int u = 0; u < R; ++u)
                if (j0 + u < cnt) x[u] = ld_nt(lane_row(base, row(j0 + u), lane));
#pragma unroll
            for (int u = 0; u < R; ++u)
                if (j0 + u < cnt) {
                    if constexpr (MODE == 0) {
                        acc += x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
                    } else {
                        x[u].x += 1u;
                        st_nt(lane_row(base, row(j0 + u), lane), x[u]);
                    }
                }
        }
    } else if constexpr (MODE == 2) {
        u32x4 a[R], b[R];
        auto load = [&](int j0, u32x4 (&x)[R]) {
#pragma unroll
            for (int u = 0; u < R; ++u)
                if (j0 + u < cnt) x[u] = ld_nt(lane_row(base, row(j0 + u), lane));
        };
        auto store = [&](int j0, u32x4 (&x)[R]) {
#pragma unroll
            for (int u = 0; u < R; ++u)
                if (j0 + u < cnt) {
                    x[u].x += 1u;
                    st_nt(lane_row(base, row(j0 + u), lane), x[u]);
                }
        };
        load(0, a);
        for (int j0 = 0; j0 < cnt; j0 += 2 * R) {
            if (j0 + R < cnt) load(j0 + R, b);
            store(j0, a);
            if (j0 + R >= cnt) break;
            if (j0 + 2 * R < cnt) load(j0 + 2 * R, a);
            store(j0 + R, b);
        }
    }
    out[static_cast<size_t>(wid) * 64 + lane] = acc;
}

// mode 3: one wave per workgroup, R rows staged in LDS per round.
template <int R>
__global__ __launch_bounds__(64) void k_rows_lds(const uint32_t* rows, int nrows, int per, unsigned char* base,
                                                 uint32_t* out) {
    __shared__ __attribute__((aligned(16))) unsigned char stage[R * kRow];
    const int lane = threadIdx.x;
    const int wid = blockIdx.x;
    const int first = wid * per;
    if (first >= nrows) return;
    const int cnt = min(per, nrows - first);
    const uint32_t my = lane < cnt ? rows[first + lane] : 0u;
    auto row = [&](int j) { return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(my), j)); };
    for (int j0 = 0; j0 < cnt; j0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u)
            if (j0 + u < cnt)
                lds_load16(lane_row(base, row(j0 + u), lane), stage + u * kRow);
        __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0): the LDS copies have landed
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < R; ++u)
            if (j0 + u < cnt) {
                u32x4 x = *reinterpret_cast<const u32x4*>(stage + u * kRow + lane * 16);
                x.x += 1u;
                st_nt(lane_row(base, row(j0 + u), lane), x);
            }
        __builtin_amdgcn_wave_barrier();
    }
    out[static_cast<size_t>(wid) * 64 + lane] = 0u;
}

__global__ __launch_bounds__(256) void k_copy(const u32x4* src, u32x4* dst, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

template <int MODE>
hipError_t launch_mode(int R, const uint32_t* rows, int nrows, int per, unsigned char* base, uint32_t* out,
                       hipStream_t s, int query, int* regs) {
    const int waves = (nrows + per - 1) / per;
    const dim3 grid((waves + 3) / 4), block(256);
    auto go = [&](auto kern) -> hipError_t {
        if (query) {
            hipFuncAttributes fa;
            hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
            *regs = fa.numRegs;
            return e;
        }
        hipLaunchKernelGGL(kern, grid, block, 0, s, rows, nrows, per, base, out);
        return hipGetLastError();
    };
    switch (R) {
        case 1: return go(k_rows<1, MODE>);
        case 2: return go(k_rows<2, MODE>);
        case 4: return go(k_rows<4, MODE>);
        case 8: return go(k_rows<8, MODE>);
        case 16: return go(k_rows<16, MODE>);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lds(int R, const uint32_t* rows, int nrows, int per, unsigned char* base, uint32_t* out,
                      hipStream_t s, int query, int* regs) {
    const int waves = (nrows + per - 1) / per;
    auto go = [&](auto kern) -> hipError_t {
        if (query) {
            hipFuncAttributes fa;
            hipError_t e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
            *regs = fa.numRegs;
            return e;
        }
        hipLaunchKernelGGL(kern, dim3(waves), dim3(64), 0, s, rows, nrows, per, base, out);
        return hipGetLastError();
    };
    switch (R) {
        case 4: return go(k_rows_lds<4>);
        case 8: return go(k_rows_lds<8>);
        case 16: return go(k_rows_lds<16>);
        case 32: return go(k_rows_lds<32>);
    }
    return hipErrorInvalidValue;
}

}  // namespace

extern "C" {

// Launches (query = 0) or reports the VGPRs of (query = 1, into *regs) the
// variant (mode, R) over nrows row ids (each < the rows of `base`), `per` per
// wavefront (1..64); out holds 64 words per wavefront.  Returns a hipError_t.
int fwpkm_probe_rows(int mode, int R, const uint32_t* rows, int nrows, int per, void* base, uint32_t* out,
                     void* stream, int query, int* regs) {
    if (per < 1 || per > 64 || nrows < 0) return hipErrorInvalidValue;
    auto* b = static_cast<unsigned char*>(base);
    hipStream_t s = static_cast<hipStream_t>(stream);
    switch (mode) {
        case 0: return launch_mode<0>(R, rows, nrows, per, b, out, s, query, regs);
        case 1: return launch_mode<1>(R, rows, nrows, per, b, out, s, query, regs);
        case 2: return launch_mode<2>(R, rows, nrows, per, b, out, s, query, regs);
        case 3: return launch_lds(R, rows, nrows, per, b, out, s, query, regs);
    }
    return hipErrorInvalidValue;
}

// Sequential copy of `bytes` (a multiple of 16) from src to dst.
int fwpkm_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_copy, dim3(8192), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return hipGetLastError();
}

}  // extern "C"
