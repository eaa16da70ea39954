// k_scatter.hip -- read-count-normalised value-row write of one chunk.
//
// With the chunk's reads sorted by slot, every value row read at least once
// is one run of equal keys.  Its gradient is the sum over the run of
// (w/H) r_t, and the write is V_i <- V_i - lr (sum) / N_read,i, N_read,i
// being the run length ("Fast-weight Product Key Memory", rainbus digest
// step 4: aggregated gradient divided by the row's read count; paperlayer.ai
// 3.3: read-count consensus; A.3: no clipping; A.4: sum reduction).  Rows
// that nobody read are never touched.
//
// The sorted list is cut into pieces of up to 64 positions (fewer when a
// small batch would leave the chip idle), one wavefront each;
// lane l owns elements [l*EPL, (l+1)*EPL) of a d_v row.  A wavefront sums
// each run of its piece in list order.  Runs inside the piece are written
// straight away; a run that crosses a piece boundary leaves per-piece
// partial sums, which k_fixup adds in piece order.  Fixed order everywhere:
// no float atomics, bitwise reproducible results.
#include "fwpkm_internal.h"

namespace fwpkm {

namespace {

// Runs whose value rows a wavefront requests at once.  Random
// read-modify-writes of 1 KiB rows reach their full rate only with many rows
// in flight; a 64-read piece holds about 60 runs at the 2^20-slot layer, so
// 16 rows per request take four round trips per wavefront, at 102 VGPRs (five
// wavefronts per SIMD).  Measured per chunk of that layer: 462 us with the
// earlier two-row pipeline, 431-435 us with 16; 10 or 12 rows (more
// wavefronts, more round trips) 451-465 us; the first residual row requested
// one or two runs ahead, or two reads of a long run per step, cost the fifth
// wavefront and did not pay.  Measured again later: 14 rows (94 VGPRs,
// five round trips) 412 -> 441 us; 20 rows (119 VGPRs, four wavefronts per
// SIMD) 412 us, the overlapped step no faster.
constexpr int kScatterRuns = 16;
// Pieces whose partials k_fixup requests at once.
constexpr int kFixupAhead = 8;

template <int STORE, int EPL>
__device__ __forceinline__ void ld_row(const void* base, size_t off, float (&x)[EPL]) {
    if constexpr (STORE == kF32) {
        const float* p = static_cast<const float*>(base) + off;
        if constexpr (EPL % 4 == 0) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4) {
                const float4 v = *reinterpret_cast<const float4*>(p + i);
                x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
            }
        } else if constexpr (EPL == 2) {
            const float2 v = *reinterpret_cast<const float2*>(p);
            x[0] = v.x; x[1] = v.y;
        } else {
            x[0] = p[0];
        }
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(base) + off;
        if constexpr (EPL == 8) {
            const uint4 v = *reinterpret_cast<const uint4*>(p);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __uint_as_float(w[i] << 16);
                x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        } else if constexpr (EPL == 4) {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xffff0000u);
            x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xffff0000u);
        } else if constexpr (EPL == 2) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
            x[0] = __uint_as_float(v << 16); x[1] = __uint_as_float(v & 0xffff0000u);
        } else {
            x[0] = bf16_to_f32(p[0]);
        }
    }
}

// A row piece in its storage form, so a load can be issued early and unpacked
// only where it is used (after other loads have been waited for).
template <int STORE, int EPL>
struct RawRow {
    static constexpr int kWords = (STORE == kF32) ? EPL : (EPL + 1) / 2;
    uint32_t w[kWords];
};

template <int STORE, int EPL>
__device__ __forceinline__ void ld_raw(const void* base, size_t off, RawRow<STORE, EPL>& x) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const unsigned char*>(base) +
                                                           off * Store<STORE>::kBytes);
    if constexpr (RawRow<STORE, EPL>::kWords % 4 == 0) {
#pragma unroll
        for (int i = 0; i < RawRow<STORE, EPL>::kWords; i += 4) {
            const uint4 v = ld16<true>(p + i);  // each row is touched once: streamed
            x.w[i] = v.x; x.w[i + 1] = v.y; x.w[i + 2] = v.z; x.w[i + 3] = v.w;
        }
    } else if constexpr (RawRow<STORE, EPL>::kWords == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        x.w[0] = v.x; x.w[1] = v.y;
    } else if constexpr (STORE == kF32 || EPL == 2) {
        x.w[0] = p[0];
    } else {
        x.w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
}

template <int STORE, int EPL>
__device__ __forceinline__ void unpack(const RawRow<STORE, EPL>& x, float (&v)[EPL]) {
    if constexpr (STORE == kF32) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) v[i] = __uint_as_float(x.w[i]);
    } else if constexpr (EPL == 1) {
        v[0] = __uint_as_float(x.w[0] << 16);
    } else {
#pragma unroll
        for (int i = 0; i < EPL / 2; ++i) {
            v[2 * i] = __uint_as_float(x.w[i] << 16);
            v[2 * i + 1] = __uint_as_float(x.w[i] & 0xffff0000u);
        }
    }
}

template <int STORE, int EPL>
__device__ __forceinline__ void st_row(void* base, size_t off, const float (&x)[EPL]) {
    if constexpr (STORE == kF32) {
        float* p = static_cast<float*>(base) + off;
        if constexpr (EPL % 4 == 0) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4)
                *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
        } else if constexpr (EPL == 2) {
            *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
        } else {
            p[0] = x[0];
        }
    } else {
        uint16_t* p = static_cast<uint16_t*>(base) + off;
        if constexpr (EPL == 8) {
            st16<true>(p, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                     pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
        } else if constexpr (EPL == 4) {
            *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
        } else if constexpr (EPL == 2) {
            *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(x[0], x[1]);
        } else {
            p[0] = static_cast<uint16_t>(f32_to_bf16(x[0]));
        }
    }
}

template <int EPL>
__device__ __forceinline__ void ld_f32(const float* p, float (&x)[EPL]) {
    if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < EPL; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(p + i);
            x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
        }
    } else if constexpr (EPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        x[0] = v.x; x[1] = v.y;
    } else {
        x[0] = p[0];
    }
}

template <int EPL>
__device__ __forceinline__ void st_f32(float* p, const float (&x)[EPL]) {
    if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < EPL; i += 4)
            *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    } else if constexpr (EPL == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    } else {
        p[0] = x[0];
    }
}

__device__ __forceinline__ size_t row_off(const ScatterArgs& a, int b, uint32_t slot, int epl) {
    return (static_cast<size_t>(b) * a.N + slot) * a.dv + static_cast<size_t>(lane_id()) * epl;
}

// V_slot <- V_slot - lr * acc / count from the row's old value v (loaded by
// the caller), one row, lanes across d_v.
template <int STORE, int EPL>
__device__ __forceinline__ void finish_row(const ScatterArgs& a, int b, uint32_t slot, int count, float (&v)[EPL],
                                           const float (&acc)[EPL]) {
    // lr / count once per row; the elements take a multiply-add
    const float sc = a.lr * __builtin_amdgcn_rcpf(static_cast<float>(count));
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = fmaf(-sc, acc[i], v[i]);
    st_row<STORE, EPL>(a.V, row_off(a, b, slot, EPL), v);
    if (a.n_read && lane_id() == 0) a.n_read[static_cast<size_t>(b) * a.N + slot] = count;
}

template <int STORE, int EPL>
__device__ __forceinline__ void apply_row(const ScatterArgs& a, int b, uint32_t slot, int count,
                                          const float (&acc)[EPL]) {
    float v[EPL];
    ld_row<STORE, EPL>(a.V, row_off(a, b, slot, EPL), v);
    finish_row<STORE, EPL>(a, b, slot, count, v, acc);
}

template <int STORE, int EPL, int R>
__global__ __launch_bounds__(256) void k_scatter(ScatterArgs a) {
    const uint32_t blk = xcd_remap(blockIdx.x, gridDim.x);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t wid = static_cast<int64_t>(blk) * 4 + wave;
    if (wid >= static_cast<int64_t>(a.B) * a.pieces) return;
    const int b = static_cast<int>(wid / a.pieces), p = static_cast<int>(wid % a.pieces);
    const int p0 = p * a.piece;
    const int pos = p0 + lane;
    const bool valid = lane < a.piece && pos < a.M;
    const uint32_t* keys = a.keys + static_cast<size_t>(b) * a.M;
    const uint32_t* vals = a.vals + static_cast<size_t>(b) * a.M;
    const uint32_t key = valid ? keys[pos] : 0xffffffffu;
    const uint32_t ent = valid ? vals[pos] : 0u;
    uint32_t prev = __shfl_up(key, 1, 64);
    uint32_t next = __shfl_down(key, 1, 64);
    if (lane == 0) prev = (p0 > 0) ? keys[p0 - 1] : 0xfffffffeu;
    if (lane == a.piece - 1) next = (pos + 1 < a.M) ? keys[pos + 1] : 0xfffffffeu;
    const bool head = valid && (pos == 0 || prev != key);
    const bool tail = valid && (pos == a.M - 1 || next != key);
    const int HK = a.H * a.k;
    const int tok = static_cast<int>(ent / static_cast<uint32_t>(HK));
    const float wv = valid ? a.w[static_cast<size_t>(b) * a.w_bstride + ent] * a.inv_h : 0.f;
    const uint64_t hb = ballot(head), tb = ballot(tail);
    const int nvalid = __popcll(ballot(valid));
    const size_t pidx = static_cast<size_t>(b) * a.pieces + p;
    if (lane == 0) {
        a.pt_start[pidx] = -1;
        a.ph_end[pidx] = -1;
    }
    // per-sequence bases; row offsets within a sequence fit 32 bits
    constexpr int ES = Store<STORE>::kBytes;
    unsigned char* Vb = static_cast<unsigned char*>(a.V) + static_cast<size_t>(b) * a.N * a.dv * ES;
    const unsigned char* rb = reinterpret_cast<const unsigned char*>(a.r + static_cast<size_t>(b) * a.Tc * a.dv);
    const uint32_t vrow = static_cast<uint32_t>(a.dv * ES), rrow = static_cast<uint32_t>(a.dv * 4);
    const uint32_t vlane = static_cast<uint32_t>(lane * EPL * ES), rlane = static_cast<uint32_t>(lane * EPL * 4);
    auto rrow_at = [&](int j) {
        const uint32_t t = static_cast<uint32_t>(__builtin_amdgcn_readlane(tok, j));
        return reinterpret_cast<const float*>(rb + (t * rrow + rlane));
    };
    auto w_at = [&](int j) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv), j)); };

    // Runs are processed in order, in batches of up to R: the value rows of
    // a batch's runs are all requested first, then each run is summed in
    // list order and its row written.
    auto run_end = [&](int s0) {
        const uint64_t tm = tb & (~0ull << s0);
        return tm != 0ull ? (__ffsll(static_cast<unsigned long long>(tm)) - 1) : nvalid - 1;
    };
    auto row_of = [&](int s0) {
        // a run wholly inside the piece writes its row; row 0 stands in for the
        // others (it is read, never written, for them)
        const uint32_t slot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key), s0));
        const int e0 = run_end(s0);
        const bool whole = ((hb >> s0) & 1ull) && ((tb >> e0) & 1ull) && slot < a.N;
        return whole ? slot : 0u;
    };
    auto finish = [&](int s0, int e, const RawRow<STORE, EPL>& vraw, const float (&x0)[EPL]) {
        const bool ends_here = (tb >> e) & 1ull;
        const bool starts_here = (hb >> s0) & 1ull;
        const uint32_t slot = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key), s0));
        const bool whole = starts_here && ends_here && slot < a.N;
        unsigned char* vp = Vb + (slot * vrow + vlane);
        const float w0 = w_at(s0);
        if (whole && e == s0) {
            // a row read once: V - lr w r
            float v[EPL];
            unpack<STORE, EPL>(vraw, v);
            const float sw = a.lr * w0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) v[i] = fmaf(-sw, x0[i], v[i]);
            st_row<STORE, EPL>(vp, 0, v);
            if (a.n_read && lane == 0) a.n_read[static_cast<size_t>(b) * a.N + slot] = 1;
            return;
        }
        float acc[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[i] = w0 * x0[i];
        for (int j = s0 + 1; j <= e; ++j) {
            float y[EPL];
            const float ww = w_at(j);
            ld_f32<EPL>(rrow_at(j), y);
#pragma unroll
            for (int i = 0; i < EPL; ++i) acc[i] = fmaf(ww, y[i], acc[i]);
        }
        if (starts_here && ends_here) {
            if (whole) {
                float v[EPL];
                unpack<STORE, EPL>(vraw, v);
                const float sc = a.lr * __builtin_amdgcn_rcpf(static_cast<float>(e - s0 + 1));
#pragma unroll
                for (int i = 0; i < EPL; ++i) v[i] = fmaf(-sc, acc[i], v[i]);
                st_row<STORE, EPL>(vp, 0, v);
                if (a.n_read && lane == 0) a.n_read[static_cast<size_t>(b) * a.N + slot] = e - s0 + 1;
            }
        } else if (!starts_here) {
            // run entering from the previous piece (it starts at lane 0)
            st_f32<EPL>(a.ph + pidx * a.dv + static_cast<size_t>(lane) * EPL, acc);
            if (lane == 0) a.ph_end[pidx] = ends_here ? p0 + e + 1 : -1;
        } else {
            // run leaving into the next piece
            st_f32<EPL>(a.pt + pidx * a.dv + static_cast<size_t>(lane) * EPL, acc);
            if (lane == 0) a.pt_start[pidx] = p0 + s0;
        }
    };

    // run starts: position 0 and every position after a run's last one
    uint64_t rem = nvalid > 0 ? (((tb << 1) | 1ull) & (nvalid == 64 ? ~0ull : ((1ull << nvalid) - 1ull))) : 0ull;
    while (rem) {
        int st[R], en[R];
        RawRow<STORE, EPL> vr[R];
        int n = 0;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (rem) {
                st[j] = __ffsll(static_cast<unsigned long long>(rem)) - 1;
                rem &= rem - 1ull;
                en[j] = run_end(st[j]);
                ld_raw<STORE, EPL>(Vb + (row_of(st[j]) * vrow + vlane), 0, vr[j]);
                n = j + 1;
            }
        }
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (j < n) {
                float r0[EPL];
                ld_f32<EPL>(rrow_at(st[j]), r0);
                finish(st[j], en[j], vr[j], r0);
            }
        }
    }
}

// Runs that cross piece boundaries: the piece a run starts in adds the
// partials of the following pieces in order, then writes the row.
template <int STORE, int EPL>
__global__ __launch_bounds__(256) void k_fixup(ScatterArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (wid >= static_cast<int64_t>(a.B) * a.pieces) return;
    const int b = static_cast<int>(wid / a.pieces), p = static_cast<int>(wid % a.pieces);
    const size_t base = static_cast<size_t>(b) * a.pieces;
    const int start = a.pt_start[base + p];
    if (start < 0) return;
    float acc[EPL];
    ld_f32<EPL>(a.pt + (base + p) * a.dv + static_cast<size_t>(lane) * EPL, acc);
    // the following pieces' partials, in piece order; a long run crosses
    // many pieces, so kFixupAhead of them are requested at a time (the sum
    // stops at the piece where the run ends)
    int end = -1;
    for (int q = p + 1; end < 0 && q < a.pieces; q += kFixupAhead) {
        float x[kFixupAhead][EPL];
        int ends[kFixupAhead];
#pragma unroll
        for (int u = 0; u < kFixupAhead; ++u)
            if (q + u < a.pieces) {
                ends[u] = a.ph_end[base + q + u];
                ld_f32<EPL>(a.ph + (base + q + u) * a.dv + static_cast<size_t>(lane) * EPL, x[u]);
            }
#pragma unroll
        for (int u = 0; u < kFixupAhead; ++u)
            if (end < 0 && q + u < a.pieces) {
#pragma unroll
                for (int i = 0; i < EPL; ++i) acc[i] += x[u][i];
                end = ends[u];
            }
    }
    if (end < 0) return;  // unreachable for a well-formed list: the last position ends a run
    const uint32_t slot = a.keys[static_cast<size_t>(b) * a.M + start];
    if (slot < a.N) apply_row<STORE, EPL>(a, b, slot, end - start, acc);
}

__global__ void k_fill_i32(int32_t* p, int64_t count, int32_t value) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t j = i; j < count; j += stride) p[j] = value;
}

// 2-D copy in 16-byte or 4-byte words (grid-stride over height x words).
template <typename W>
__global__ void k_copy2d(unsigned char* dst, int64_t dpitch, const unsigned char* src, int64_t spitch,
                         int64_t words, int64_t height) {
    const int64_t total = words * height;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t y = i / words, x = i - y * words;
        *reinterpret_cast<W*>(dst + y * dpitch + x * static_cast<int64_t>(sizeof(W))) =
            *reinterpret_cast<const W*>(src + y * spitch + x * static_cast<int64_t>(sizeof(W)));
    }
}

template <int STORE, int EPL>
hipError_t scatter_t(const ScatterArgs& a, hipStream_t s) {
    const int64_t waves = static_cast<int64_t>(a.B) * a.pieces;
    const unsigned grid = static_cast<unsigned>((waves + 3) / 4);
    hipLaunchKernelGGL((k_scatter<STORE, EPL, kScatterRuns>), dim3(grid), dim3(256), 0, s, a);
    hipLaunchKernelGGL((k_fixup<STORE, EPL>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int STORE>
hipError_t scatter_s(const ScatterArgs& a, hipStream_t s) {
    switch (a.dv / 64) {
        case 1: return scatter_t<STORE, 1>(a, s);
        case 2: return scatter_t<STORE, 2>(a, s);
        case 4: return scatter_t<STORE, 4>(a, s);
        case 8: return scatter_t<STORE, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scatter(const ScatterArgs& a, int store, hipStream_t s) {
    return store == kBF16 ? scatter_s<kBF16>(a, s) : scatter_s<kF32>(a, s);
}

hipError_t launch_fill_i32(int32_t* p, int64_t count, int32_t value, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, count, value);
    return hipGetLastError();
}

hipError_t launch_copy2d(void* dst, int64_t dpitch, const void* src, int64_t spitch, int64_t width_bytes,
                         int64_t height, hipStream_t s) {
    if (width_bytes <= 0 || height <= 0) return hipSuccess;
    if (width_bytes % 4) return hipErrorInvalidValue;
    auto* d = static_cast<unsigned char*>(dst);
    const auto* sp = static_cast<const unsigned char*>(src);
    const bool wide = width_bytes % 16 == 0 && dpitch % 16 == 0 && spitch % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(d) % 16 == 0 && reinterpret_cast<uintptr_t>(sp) % 16 == 0;
    const int64_t words = width_bytes / (wide ? 16 : 4);
    int64_t blocks = (words * height + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (wide)
        hipLaunchKernelGGL(k_copy2d<uint4>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, d, dpitch, sp,
                           spitch, words, height);
    else
        hipLaunchKernelGGL(k_copy2d<uint32_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, d, dpitch, sp,
                           spitch, words, height);
    return hipGetLastError();
}

}  // namespace fwpkm
