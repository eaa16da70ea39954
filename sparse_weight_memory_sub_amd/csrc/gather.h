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
// gather was timed alone.  The chunk gather streams (non-temporal loads) the
// rows of the sequences that would leave the cache before the write reaches
// them (GatherArgs::keep_b0): at that layer gather 214 -> 204 us, the write
// unchanged, the overlapped step 7.71 -> 7.62 ms.
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
template <int STORE, int EPL, int ROWS, bool NT = kGatherNt>
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
            ldrow<STORE, EPL, NT>(a.V, vb + static_cast<size_t>(s) * a.dv + col, x[u]);
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
        ldrow<STORE, EPL, NT>(a.V, vb + static_cast<size_t>(s) * a.dv + col, x);
#pragma unroll
        for (int i = 0; i < EPL; ++i) acc[i] = fmaf(ww, x[i], acc[i]);
    }
}

// The loads of a token's epilogue: g_t, v_t (for o) and the raw target (for
// the residual).  Apart from the stores so that a caller can request them
// before the weighted sum is known.
template <int EPL>
struct FinishIn {
    float gt;
    float vt[EPL];
    float y[EPL];
};

template <int STORE, int EPL>
__device__ __forceinline__ void finish_load(const GatherArgs& a, int b, int t, int lane, FinishIn<EPL>& in) {
    const size_t col = static_cast<size_t>(lane) * EPL;
    in.gt = a.g[static_cast<size_t>(b) * a.g_bstride + t];
    if (a.o) ldrow<STORE, EPL>(a.v, static_cast<size_t>(b) * a.v_bstride + static_cast<size_t>(t) * a.dv + col, in.vt);
    if (a.r && t < a.n_tgt) {
        if (a.tgt_last && t == a.Tc - 1)
            ldrow<STORE, EPL>(a.tgt_last, static_cast<size_t>(b) * a.tgt_last_bstride + col, in.y);
        else
            ldrow<STORE, EPL>(a.tgt, static_cast<size_t>(b) * a.tgt_bstride + static_cast<size_t>(t) * a.dv + col, in.y);
    }
}

// Everything after the weighted sum but the stream's copies: v_hat, o and
// the residual.
template <int EPL>
__device__ __forceinline__ void finish_store(const GatherArgs& a, int b, int t, int lane, const float (&tot)[EPL],
                                             FinishIn<EPL>& in) {
    const size_t col = static_cast<size_t>(lane) * EPL;
    const float Hf = static_cast<float>(a.H);
    float vh[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) vh[i] = tot[i] / Hf;
    const float gt = in.gt;
    if (a.o) {
        float o[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) o[i] = gt * vh[i] + (1.f - gt) * in.vt[i];
        const size_t oo = static_cast<size_t>(b) * a.o_bstride + static_cast<size_t>(t) * a.dv + col;
        stf<EPL>(a.o + oo, o);
        if (a.vhat) stf<EPL>(a.vhat + oo, vh);
    }
    if (a.vhat2)
        stf<EPL>(a.vhat2 + static_cast<size_t>(b) * a.vhat2_bstride + static_cast<size_t>(t) * a.dv + col, vh);
    if (a.r && t < a.n_tgt) {
        if (a.znorm) zscore<EPL>(in.y, a.dv, a.znorm_eps);
        float rr[EPL];
        const float gw = a.gate_w ? gt : 1.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) rr[i] = gw * (vh[i] - in.y[i]);
        stf<EPL>(a.r + (static_cast<size_t>(b) * a.Tc + t) * a.dv + col, rr);
    }
}

// A stream's copies of token t into the pending chunk: q, g, and v as the
// target of slot t + ptgt_shift (none below 0).  The 16-byte pieces of the
// two rows (q first) are numbered 0 .. pending_pieces - 1; `first` and
// `step` pick the pieces of the caller (a lane of a wavefront, or a thread
// of a workgroup).
template <int STORE>
__device__ __forceinline__ int pending_qpieces(const GatherArgs& a) {
    return a.qrow * Store<STORE>::kBytes / 16;
}

template <int STORE>
__device__ __forceinline__ int pending_pieces(const GatherArgs& a, int t) {
    return pending_qpieces<STORE>(a) + (t + a.ptgt_shift >= 0 ? a.dv * Store<STORE>::kBytes / 16 : 0);
}

template <int STORE>
__device__ __forceinline__ uint4* pending_dst(const GatherArgs& a, int b, int t, int w) {
    constexpr int ES = Store<STORE>::kBytes;
    const int nq = pending_qpieces<STORE>(a);
    if (w < nq)
        return reinterpret_cast<uint4*>(static_cast<unsigned char*>(a.pq) +
                                        (static_cast<size_t>(b) * a.pq_bstride + static_cast<size_t>(t) * a.qrow) * ES) + w;
    return reinterpret_cast<uint4*>(static_cast<unsigned char*>(a.ptgt) +
                                    (static_cast<size_t>(b) * a.ptgt_bstride + static_cast<size_t>(t + a.ptgt_shift) * a.dv) * ES) +
           (w - nq);
}

template <int STORE>
__device__ __forceinline__ const uint4* pending_src(const GatherArgs& a, int b, int t, int w) {
    constexpr int ES = Store<STORE>::kBytes;
    const int nq = pending_qpieces<STORE>(a);
    if (w < nq)
        return reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(a.q) +
                                              (static_cast<size_t>(b) * a.q_bstride + static_cast<size_t>(t) * a.qrow) * ES) + w;
    return reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(a.v) +
                                          (static_cast<size_t>(b) * a.v_bstride + static_cast<size_t>(t) * a.dv) * ES) +
           (w - nq);
}

template <int STORE>
__device__ __forceinline__ void pending_copy(const GatherArgs& a, int b, int t, int first, int step) {
    const int n = pending_pieces<STORE>(a, t);
    for (int w = first; w < n; w += step) *pending_dst<STORE>(a, b, t, w) = *pending_src<STORE>(a, b, t, w);
}

// Everything after the weighted sum: v_hat, o, the residual and, for a
// stream, the copies of the token's inputs into the pending chunk.
template <int STORE, int EPL>
__device__ __forceinline__ void gather_finish(const GatherArgs& a, int b, int t, int lane, const float (&tot)[EPL]) {
    FinishIn<EPL> in;
    finish_load<STORE, EPL>(a, b, t, lane, in);
    finish_store<EPL>(a, b, t, lane, tot, in);
    if (a.pq) {
        if (lane == 0) a.pg[static_cast<size_t>(b) * a.pg_bstride + t] = in.gt;
        pending_copy<STORE>(a, b, t, lane, 64);
    }
}

// gather_part for bf16 rows with all ROWS rows of a round held as their raw
// bf16 words until their multiply-adds (half the registers of widened
// rows), so a part of 16 entries is one round trip where registers are
// few.  The same multiply-adds in the same order, so the same bits.
template <int EPL>
struct Bf16Row {
    uint32_t w[(EPL + 1) / 2];
};

template <int EPL, bool NT = kGatherNt>
__device__ __forceinline__ void ld_bf16_row(const void* base, size_t off, Bf16Row<EPL>& r) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    if constexpr (EPL == 8) {
        const uint4 v = ld16<NT>(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else if constexpr (EPL == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        r.w[0] = v.x; r.w[1] = v.y;
    } else if constexpr (EPL == 2) {
        r.w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
        r.w[0] = static_cast<uint32_t>(p[0]) << 16;
    }
}

template <int EPL>
__device__ __forceinline__ void fma_bf16_row(float ww, const Bf16Row<EPL>& r, float (&acc)[EPL]) {
    if constexpr (EPL == 1) {
        acc[0] = fmaf(ww, __uint_as_float(r.w[0]), acc[0]);
    } else {
#pragma unroll
        for (int i = 0; i < EPL / 2; ++i) {
            acc[2 * i] = fmaf(ww, __uint_as_float(r.w[i] << 16), acc[2 * i]);
            acc[2 * i + 1] = fmaf(ww, __uint_as_float(r.w[i] & 0xffff0000u), acc[2 * i + 1]);
        }
    }
}

// A row's lane share as loaded (fp32 words, or raw bf16 words), widened
// only where it is used.
template <int STORE, int EPL>
struct RawRow;
template <int EPL>
struct RawRow<kF32, EPL> {
    float x[EPL];
};
template <int EPL>
struct RawRow<kBF16, EPL> {
    Bf16Row<EPL> r;
};

template <int STORE, int EPL>
__device__ __forceinline__ void ld_raw_row(const void* base, size_t off, RawRow<STORE, EPL>& r) {
    if constexpr (STORE == kF32) ldrow<kF32, EPL>(base, off, r.x);
    else ld_bf16_row<EPL>(base, off, r.r);
}

template <int STORE, int EPL>
__device__ __forceinline__ void widen_raw_row(const RawRow<STORE, EPL>& r, float (&x)[EPL]) {
    if constexpr (STORE == kF32) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) x[i] = r.x[i];
    } else if constexpr (EPL == 1) {
        x[0] = __uint_as_float(r.r.w[0]);
    } else {
#pragma unroll
        for (int i = 0; i < EPL / 2; ++i) {
            x[2 * i] = __uint_as_float(r.r.w[i] << 16);
            x[2 * i + 1] = __uint_as_float(r.r.w[i] & 0xffff0000u);
        }
    }
}

template <int EPL, int ROWS, bool NT = kGatherNt>
__device__ __forceinline__ void gather_part_held(const GatherArgs& a, size_t vb, size_t col, int32_t sl, float wt,
                                                 int base, int cnt, float (&acc)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
    int j = 0;
    for (; j + ROWS <= cnt; j += ROWS) {
        Bf16Row<EPL> x[ROWS];
        float ww[ROWS];
#pragma unroll
        for (int u = 0; u < ROWS; ++u) {
            const int s = __builtin_amdgcn_readlane(sl, base + j + u);
            ww[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), base + j + u));
            ld_bf16_row<EPL, NT>(a.V, vb + static_cast<size_t>(s) * a.dv + col, x[u]);
        }
#pragma unroll
        for (int u = 0; u < ROWS; ++u) fma_bf16_row<EPL>(ww[u], x[u], acc);
    }
    for (; j < cnt; ++j) {
        Bf16Row<EPL> x;
        const int s = __builtin_amdgcn_readlane(sl, base + j);
        const float ww = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt), base + j));
        ld_bf16_row<EPL, NT>(a.V, vb + static_cast<size_t>(s) * a.dv + col, x);
        fma_bf16_row<EPL>(ww, x, acc);
    }
}

// One token's read by one workgroup of at least ceil(H*k / kGatherPart)
// wavefronts, one per part; the parts meet in `part` (LDS) and the first
// wavefront folds them in part order, so the result is bitwise that of a
// single wavefront summing the parts in order.  Every thread of the
// workgroup must call it (it holds a barrier).  With `pre`, the first
// wavefront's epilogue inputs were loaded by the caller and the stream's
// copies are the caller's too; bf16 rows are then read in one round trip
// per part.
template <int STORE, int EPL>
__device__ __forceinline__ void gather_token_split(const GatherArgs& a, int64_t tok, float (*part)[512],
                                                   FinishIn<EPL>* pre = nullptr) {
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
        const size_t vb = static_cast<size_t>(b) * static_cast<size_t>(a.N) * a.dv;
        float acc[EPL];
        if (STORE == kBF16 && pre)
            gather_part_held<EPL, kGatherPart>(a, vb, col, sl, wt, 0, cnt, acc);
        else
            gather_part<STORE, EPL, 8>(a, vb, col, sl, wt, 0, cnt, acc);
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
    if (pre) finish_store<EPL>(a, b, t, lane, tot, *pre);
    else gather_finish<STORE, EPL>(a, b, t, lane, tot);
}

}  // namespace fwpkm
