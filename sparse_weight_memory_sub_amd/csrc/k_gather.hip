// k_gather.hip -- weighted read of the selected value rows, gated output and
// the memorisation residual.
//
// Read and output (rainbus digest of "Fast-weight Product Key Memory",
// steps 2-3): v_hat_t = (1/H) sum_h sum_j w V[idx], o_t = g_t v_hat_t +
// (1 - g_t) v_t.  Residual of the gated reconstruction loss (digest step 4;
// paperlayer.ai A.1, A.3, A.5): r_t = g_t (v_hat_t - y_t) with y_t the
// z-scored lookahead target.
//
// One wavefront per token; lane l owns elements [l*EPL, (l+1)*EPL) of every
// d_v-row, so each row read is one coalesced d_v*elem_bytes transaction of
// the wavefront.  Rows are fetched eight at a time to keep several HBM reads
// in flight per wavefront.
#include "fwpkm_internal.h"

namespace fwpkm {

namespace {

template <int STORE, int EPL, bool NT = false>
__device__ __forceinline__ void ldrow(const void* base, size_t off, float (&x)[EPL]) {
    if constexpr (STORE == kF32) {
        const float* p = static_cast<const float*>(base) + off;
        if constexpr (EPL % 4 == 0) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4) {
                const uint4 v = ld16<NT>(p + i);
                x[i] = __uint_as_float(v.x); x[i + 1] = __uint_as_float(v.y);
                x[i + 2] = __uint_as_float(v.z); x[i + 3] = __uint_as_float(v.w);
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
            const uint4 v = ld16<NT>(p);
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

template <int EPL>
__device__ __forceinline__ void stf(float* p, const float (&x)[EPL]) {
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

// y <- (y - mean) / sqrt(var + eps), statistics over the d_v elements of the
// row spread across the wavefront (population variance).
template <int EPL>
__device__ __forceinline__ void zscore(float (&y)[EPL], int dv, float eps) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) s += y[i];
    const float mean = wave_sum(s) / static_cast<float>(dv);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float d = y[i] - mean;
        q = fmaf(d, d, q);
    }
    const float var = wave_sum(q) / static_cast<float>(dv);
    const float inv = 1.f / sqrtf(var + eps);
#pragma unroll
    for (int i = 0; i < EPL; ++i) y[i] = (y[i] - mean) * inv;
}

template <int STORE, int EPL>
__global__ __launch_bounds__(256) void k_gather(GatherArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (tok >= static_cast<int64_t>(a.B) * a.Tc) return;
    const int b = static_cast<int>(tok / a.Tc), t = static_cast<int>(tok % a.Tc);
    const int HK = a.H * a.k;
    const size_t ib = static_cast<size_t>(b) * a.iw_bstride + static_cast<size_t>(t) * HK;
    // up to 4*64 (slot, weight) entries, entry e held by lane e % 64, register e / 64
    int32_t sl[4];
    float wt[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = r * 64 + lane;
        sl[r] = (e < HK) ? a.idx[ib + e] : 0;
        wt[r] = (e < HK) ? a.w[ib + e] : 0.f;
    }
    const size_t vb = static_cast<size_t>(b) * static_cast<size_t>(a.N) * a.dv;
    const size_t col = static_cast<size_t>(lane) * EPL;
    float acc[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = 0.f;

#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int cnt = min(64, HK - r * 64);
        if (cnt <= 0) break;
        int j = 0;
        for (; j + 8 <= cnt; j += 8) {
            float x[8][EPL];
            float ww[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s = __builtin_amdgcn_readlane(sl[r], j + u);
                ww[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt[r]), j + u));
                ldrow<STORE, EPL, true>(a.V, vb + static_cast<size_t>(s) * a.dv + col, x[u]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int i = 0; i < EPL; ++i) acc[i] = fmaf(ww[u], x[u][i], acc[i]);
        }
        for (; j < cnt; ++j) {
            float x[EPL];
            const int s = __builtin_amdgcn_readlane(sl[r], j);
            const float ww = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt[r]), j));
            ldrow<STORE, EPL, true>(a.V, vb + static_cast<size_t>(s) * a.dv + col, x);
#pragma unroll
            for (int i = 0; i < EPL; ++i) acc[i] = fmaf(ww, x[i], acc[i]);
        }
    }
    const float Hf = static_cast<float>(a.H);
    float vh[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) vh[i] = acc[i] / Hf;

    const float gt = a.g[static_cast<size_t>(b) * a.g_bstride + t];
    if (a.o) {
        float vt[EPL], o[EPL];
        ldrow<STORE, EPL>(a.v, static_cast<size_t>(b) * a.v_bstride + static_cast<size_t>(t) * a.dv + col, vt);
#pragma unroll
        for (int i = 0; i < EPL; ++i) o[i] = gt * vh[i] + (1.f - gt) * vt[i];
        const size_t oo = static_cast<size_t>(b) * a.o_bstride + static_cast<size_t>(t) * a.dv + col;
        stf<EPL>(a.o + oo, o);
        if (a.vhat) stf<EPL>(a.vhat + oo, vh);
    }
    if (a.vhat2)
        stf<EPL>(a.vhat2 + static_cast<size_t>(b) * a.vhat2_bstride + static_cast<size_t>(t) * a.dv + col, vh);
    if (a.r && t < a.n_tgt) {
        float y[EPL];
        if (a.tgt_last && t == a.Tc - 1)
            ldrow<STORE, EPL>(a.tgt_last, static_cast<size_t>(b) * a.tgt_last_bstride + col, y);
        else
            ldrow<STORE, EPL>(a.tgt, static_cast<size_t>(b) * a.tgt_bstride + static_cast<size_t>(t) * a.dv + col, y);
        if (a.znorm) zscore<EPL>(y, a.dv, a.znorm_eps);
        float rr[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) rr[i] = gt * (vh[i] - y[i]);
        stf<EPL>(a.r + (static_cast<size_t>(b) * a.Tc + t) * a.dv + col, rr);
    }
}

template <int STORE, int EPL>
__global__ __launch_bounds__(256) void k_resid(ResidArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (tok >= static_cast<int64_t>(a.B) * a.n_tgt) return;
    const int b = static_cast<int>(tok / a.n_tgt), t = static_cast<int>(tok % a.n_tgt);
    const size_t col = static_cast<size_t>(lane) * EPL;
    float y[EPL], vh[EPL];
    ldrow<STORE, EPL>(a.tgt, static_cast<size_t>(b) * a.tgt_bstride + static_cast<size_t>(t) * a.dv + col, y);
    if (a.znorm) zscore<EPL>(y, a.dv, a.znorm_eps);
    ldrow<kF32, EPL>(a.vhat, static_cast<size_t>(b) * a.vhat_bstride + static_cast<size_t>(t) * a.dv + col, vh);
    const float gt = a.g[static_cast<size_t>(b) * a.g_bstride + t];
    float rr[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) rr[i] = gt * (vh[i] - y[i]);
    stf<EPL>(a.r + (static_cast<size_t>(b) * a.Tc + t) * a.dv + col, rr);
}

template <int STORE, int EPL>
hipError_t gather_t(const GatherArgs& a, hipStream_t s) {
    const int64_t toks = static_cast<int64_t>(a.B) * a.Tc;
    const unsigned grid = static_cast<unsigned>((toks + 3) / 4);
    hipLaunchKernelGGL((k_gather<STORE, EPL>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int STORE, int EPL>
hipError_t resid_t(const ResidArgs& a, hipStream_t s) {
    const int64_t toks = static_cast<int64_t>(a.B) * a.n_tgt;
    const unsigned grid = static_cast<unsigned>((toks + 3) / 4);
    hipLaunchKernelGGL((k_resid<STORE, EPL>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int STORE>
hipError_t gather_s(const GatherArgs& a, hipStream_t s) {
    switch (a.dv / 64) {
        case 1: return gather_t<STORE, 1>(a, s);
        case 2: return gather_t<STORE, 2>(a, s);
        case 4: return gather_t<STORE, 4>(a, s);
        case 8: return gather_t<STORE, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int STORE>
hipError_t resid_s(const ResidArgs& a, hipStream_t s) {
    switch (a.dv / 64) {
        case 1: return resid_t<STORE, 1>(a, s);
        case 2: return resid_t<STORE, 2>(a, s);
        case 4: return resid_t<STORE, 4>(a, s);
        case 8: return resid_t<STORE, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, int store, hipStream_t s) {
    return store == kBF16 ? gather_s<kBF16>(a, s) : gather_s<kF32>(a, s);
}

hipError_t launch_resid(const ResidArgs& a, int store, hipStream_t s) {
    return store == kBF16 ? resid_s<kBF16>(a, s) : resid_s<kF32>(a, s);
}

}  // namespace fwpkm
