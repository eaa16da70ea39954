// gather.h -- device parts of the weighted value read shared by the gather
// kernels and the fused decode selection: the sum of a part of a token's
// (slot, weight) entries, the gated output / residual / pending-chunk copies
// of a token, and the whole read of one token by one workgroup.
//
// Lane l owns elements [l*EPL, (l+1)*EPL) of every d_v-row, so each row read
// is one coalesced d_v*elem_bytes transaction of a wavefront.  A token's H*k
// rows are summed in parts of kGatherPart consecutive entries, each part in
// entry order, and the parts are added in order.
#pragma once

#include "rows.h"

// The value rows are read with ordinary (cache-allocating) loads: the chunk's
// value write, which follows, reads the same rows, and part of them is then
// still in the 256 MB last-level cache.  Measured per chunk of the 2^20-slot
// layer (serialized timing): gather 198 -> 215 us, write 440 -> 408 us, with
// the overlapped step unchanged; non-temporal loads had been chosen when the
// gather was timed alone.
constexpr bool kGatherNt = false;

namespace fwpkm {

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

// Rows [e0, e0 + cnt) of the token's H*k (slot, weight) entries, summed in
// entry order into acc (this lane's EPL columns).  Entry e0 + j is held by
// lane `base + j` of the wavefront's (sl, wt) registers.  Rows are fetched
// eight at a time so several HBM reads are in flight.
// ROWS value rows in flight per wavefront: 16 for the chunk gather (its
// wavefronts share the chip with the key path; 8.15 -> 8.09 ms per step at
// million), 8 for the few-token gather (16 makes decode's 9.8 -> 15.9 us).
// The rows of a part are summed in the same order either way.
template <int STORE, int EPL, int ROWS>
__device__ __forceinline__ void gather_part(const GatherArgs& a, size_t vb, size_t col, int32_t sl, float wt, int base,
                                            int cnt, float (&acc)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
    int j = 0;
    for (; j + ROWS <= cnt; j += ROWS) {
        float x[ROWS][EPL];
        float ww[ROWS];
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int s = __builtin_amdgcn_readlane(sl, base + j + u);
            ww[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), base + j + u));
            ldrow<STORE, EPL, kGatherNt>(a.V, vb + static_cast<size_t>(s) * a.dv + col, x[u]);
        }
#pragma unroll
        for (int u = 0; u < ROWS; ++u)
#pragma unroll
            for (int i = 0; i < EPL; ++i) acc[i] = fmaf(ww[u], x[u][i], acc[i]);
    }
    for (; j < cnt; ++j) {
        float x[EPL];
        const int s = __builtin_amdgcn_readlane(sl, base + j);
        const float ww = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), base + j));
        ldrow<STORE, EPL, kGatherNt>(a.V, vb + static_cast<size_t>(s) * a.dv + col, x);
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[i] = fmaf(ww, x[i], acc[i]);
    }
}

// Row of `bytes` (a multiple of 16) from src to dst by the whole wavefront.
__device__ __forceinline__ void copy_row16(void* dst, const void* src, int bytes, int lane) {
    for (int w = lane; w < bytes / 16; w += 64)
        reinterpret_cast<uint4*>(dst)[w] = reinterpret_cast<const uint4*>(src)[w];
}

// Everything after the weighted sum: v_hat, o, the residual and, for a
// stream, the copies of the token's inputs into the pending chunk.
template <int STORE, int EPL>
__device__ __forceinline__ void gather_finish(const GatherArgs& a, int b, int t, int lane, const float (&tot)[EPL]) {
    constexpr int ES = Store<STORE>::kBytes;
    const size_t col = static_cast<size_t>(lane) * EPL;
    const float Hf = static_cast<float>(a.H);
    float vh[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) vh[i] = tot[i] / Hf;

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
        const float gw = a.gate_w ? gt : 1.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) rr[i] = gw * (vh[i] - y[i]);
        stf<EPL>(a.r + (static_cast<size_t>(b) * a.Tc + t) * a.dv + col, rr);
    }
    if (a.pq) {
        const int qbytes = a.qrow * ES;
        copy_row16(static_cast<unsigned char*>(a.pq) + (static_cast<size_t>(b) * a.pq_bstride + static_cast<size_t>(t) * a.qrow) * ES,
                   static_cast<const unsigned char*>(a.q) + (static_cast<size_t>(b) * a.q_bstride + static_cast<size_t>(t) * a.qrow) * ES,
                   qbytes, lane);
        if (lane == 0) a.pg[static_cast<size_t>(b) * a.pg_bstride + t] = gt;
        const int slot = t + a.ptgt_shift;
        if (slot >= 0)
            copy_row16(static_cast<unsigned char*>(a.ptgt) + (static_cast<size_t>(b) * a.ptgt_bstride + static_cast<size_t>(slot) * a.dv) * ES,
                       static_cast<const unsigned char*>(a.v) + (static_cast<size_t>(b) * a.v_bstride + static_cast<size_t>(t) * a.dv) * ES,
                       a.dv * ES, lane);
    }
}

// One wavefront per token: the parts of kGatherPart entries are summed in
// turn and folded into the total in part order.
// One token's read by one workgroup of at least ceil(H*k / kGatherPart)
// wavefronts, one per part; the parts meet in `part` (LDS) and the first
// wavefront folds them in part order, so the result is bitwise that of a
// single wavefront summing the parts in order.  Every thread of the
// workgroup must call it (it holds a barrier).
template <int STORE, int EPL>
__device__ __forceinline__ void gather_token_split(const GatherArgs& a, int64_t tok, float (*part)[512]) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int b = static_cast<int>(tok / a.Tc), t = static_cast<int>(tok % a.Tc);
    const int HK = a.H * a.k;
    const int nparts = (HK + kGatherPart - 1) / kGatherPart;
    const size_t col = static_cast<size_t>(lane) * EPL;
    if (wave < nparts) {
        const int e0 = wave * kGatherPart;
        const int cnt = min(kGatherPart, HK - e0);
        const size_t ib = static_cast<size_t>(b) * a.iw_bstride + static_cast<size_t>(t) * HK + e0;
        const int32_t sl = (lane < cnt) ? a.idx[ib + lane] : 0;
        const float wt = (lane < cnt) ? a.w[ib + lane] : 0.f;
        float acc[EPL];
        gather_part<STORE, EPL, 8>(a, static_cast<size_t>(b) * static_cast<size_t>(a.N) * a.dv, col, sl, wt, 0, cnt, acc);
#pragma unroll
        for (int i = 0; i < EPL; ++i) part[wave][col + i] = acc[i];
    }
    __syncthreads();
    if (wave != 0) return;
    float tot[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) tot[i] = part[0][col + i];
    for (int p = 1; p < nparts; ++p)
#pragma unroll
        for (int i = 0; i < EPL; ++i) tot[i] = tot[i] + part[p][col + i];
    gather_finish<STORE, EPL>(a, b, t, lane, tot);
}

}  // namespace fwpkm
