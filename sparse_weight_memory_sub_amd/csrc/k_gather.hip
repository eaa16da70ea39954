// k_gather.hip -- weighted read of the selected value rows, gated output and
// the memorisation residual.
//
// Read and output (rainbus digest of "Fast-weight Product Key Memory",
// steps 2-3): v_hat_t = (1/H) sum_h sum_j w V[idx], o_t = g_t v_hat_t +
// (1 - g_t) v_t.  Residual of the gated reconstruction loss (digest step 4;
// paperlayer.ai A.1, A.3, A.5): r_t = g_t (v_hat_t - y_t) with y_t the
// z-scored lookahead target (r_t = v_hat_t - y_t with the gate weighting off).
//
// Lane l owns elements [l*EPL, (l+1)*EPL) of every d_v-row, so each row read
// is one coalesced d_v*elem_bytes transaction of a wavefront.  A token's H*k
// rows are summed in parts of kGatherPart consecutive entries, each part in
// entry order, and the parts are added in order: one wavefront per token
// for large batches (k_gather), one wavefront per part when the tokens are
// too few to fill the chip (k_gather_split, decode); both give the same bits.
// HELD (bf16 storage) keeps a round's rows as their raw words until their
// multiply-adds: fewer registers and more wavefronts per SIMD, the same bits.
#include "gather.h"

namespace fwpkm {

namespace {

template <int STORE, int EPL, bool HELD>
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
    // rows the value write will find in the last-level cache are read into
    // it; the others stream (gather_keep_from)
    const bool keep = b >= a.keep_b0;
    float tot[EPL];
#pragma unroll
    for (int p = 0; p < 256 / kGatherPart; ++p) {
        const int e0 = p * kGatherPart;
        if (e0 >= HK) break;
        float acc[EPL];
        if constexpr (HELD) {
            if (keep)
                gather_part_held<EPL, 16, false>(a, vb, col, sl[e0 / 64], wt[e0 / 64], e0 % 64,
                                                 min(kGatherPart, HK - e0), acc);
            else
                gather_part_held<EPL, 16, true>(a, vb, col, sl[e0 / 64], wt[e0 / 64], e0 % 64,
                                                min(kGatherPart, HK - e0), acc);
        } else {
            if (keep)
                gather_part<STORE, EPL, 16, false>(a, vb, col, sl[e0 / 64], wt[e0 / 64], e0 % 64,
                                                   min(kGatherPart, HK - e0), acc);
            else
                gather_part<STORE, EPL, 16, true>(a, vb, col, sl[e0 / 64], wt[e0 / 64], e0 % 64,
                                                  min(kGatherPart, HK - e0), acc);
        }
#pragma unroll
        for (int i = 0; i < EPL; ++i) tot[i] = (p == 0) ? acc[i] : tot[i] + acc[i];
    }
    gather_finish<STORE, EPL>(a, b, t, lane, tot);
}

// The same sums for few tokens: one workgroup per token, one wavefront per
// part (gather_token_split), the same bits as k_gather.
template <int STORE, int EPL>
__global__ __launch_bounds__(64 * (256 / kGatherPart)) void k_gather_split(GatherArgs a) {
    __shared__ float part[256 / kGatherPart][512];
    gather_token_split<STORE, EPL>(a, blockIdx.x, part);
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
    const float gt = a.gate_w ? a.g[static_cast<size_t>(b) * a.g_bstride + t] : 1.f;
    float rr[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) rr[i] = gt * (vh[i] - y[i]);
    stf<EPL>(a.r + (static_cast<size_t>(b) * a.Tc + t) * a.dv + col, rr);
}

template <int STORE, int EPL>
hipError_t gather_t(const GatherArgs& a, hipStream_t s) {
    const int64_t toks = static_cast<int64_t>(a.B) * a.Tc;
    if (toks < kGatherSplitBelow) {
        const int nparts = (a.H * a.k + kGatherPart - 1) / kGatherPart;
        hipLaunchKernelGGL((k_gather_split<STORE, EPL>), dim3(static_cast<unsigned>(toks)), dim3(64 * nparts), 0, s, a);
    } else {
        const unsigned grid = static_cast<unsigned>((toks + 3) / 4);
        if (STORE == kBF16 && a.held)
            hipLaunchKernelGGL((k_gather<STORE, EPL, STORE == kBF16>), dim3(grid), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_gather<STORE, EPL, false>), dim3(grid), dim3(256), 0, s, a);
    }
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
