// k_sweep.hip -- sub-key scoring sweep of one 16-token tile against every
// sub-key of both half codebooks of one (sequence, head).
//
// Scoring ("Fast-weight Product Key Memory": paperlayer.ai 2.2 and A.2,
// rainbus digest step 2): the query is split into halves and each half is
// compared with every sub-key of its codebook by squared Euclidean distance,
// taken here as the contraction ||q||^2 + ||K_i||^2 - 2 q.K_i on the matrix
// cores (16x16 MFMA tiles over 32-wide k-blocks).  The distances of the
// tile, e = eps + max(d, 0), stay in LDS and feed, depending on the mode:
//
//  kSweepSelect   top-k' smallest e per half (radix select on the fp32 bit
//                 pattern, ties to the lower sub-key index), then the top-k
//                 of the product candidates ordered by P = e1*e2 (ties to the
//                 lower slot id i*n + j), weights (1/P) / sum(1/P) -- the
//                 softmax of the pair scores s1 + s2 = -log P.
//  kSweepStats    per-tile sums over tokens of p_ti = (1/e_ti) / Z_t,
//                 Z_t = sum_i 1/e_ti (softmax of s over all sub-keys), the
//                 pieces of the chunk's marginal usage pbar (digest step 5,
//                 paperlayer.ai 3.4).
//  kSweepRowStat  Z_t and m_t = sum_i p_ti log pbar_i, the row statistic of
//                 the entropy gradient.
#include "mfma_frag.h"

namespace fwpkm {

namespace {

constexpr int kNplMax = 16;  // sub-keys per lane in a row scan: n <= 1024

// Ascending bitonic sort of one 64-bit key per lane across the wavefront.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), m, 64);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), m, 64);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Sorts R*64 keys held as element p = r*64 + lane, ascending.
template <int R>
__device__ __forceinline__ void bitonic_sort(uint64_t (&x)[R]) {
    const int lane = lane_id();
#pragma unroll
    for (int size = 2; size <= 64 * R; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= 64) {
                const int rs = stride >> 6;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if ((r & rs) == 0) {
                        const int r2 = r | rs;
                        const int p = r * 64 + lane;
                        const bool up = (p & size) == 0;
                        const uint64_t a = x[r], b = x[r2];
                        const bool sw = up ? (a > b) : (a < b);
                        x[r] = sw ? b : a;
                        x[r2] = sw ? a : b;
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint64_t y = shfl_xor_u64(x[r], stride);
                    const int p = r * 64 + lane;
                    const bool up = (p & size) == 0;
                    const bool lower = (lane & stride) == 0;
                    const bool keep_min = (lower == up);
                    const uint64_t mn = x[r] < y ? x[r] : y;
                    const uint64_t mx = x[r] < y ? y : x[r];
                    x[r] = keep_min ? mn : mx;
                }
            }
        }
    }
}

// Top-kh smallest of the row u[j] (element index j*64 + lane, bit patterns
// of non-negative floats, +inf padding) with ties to the lower index.
// Writes the kh winners sorted ascending by (value, index) to out_e/out_i.
__device__ void wave_select(const uint32_t (&u)[kNplMax], int npl, int kh,
                            uint32_t* hist, float* out_e, int* out_i) {
    const int lane = lane_id();
    uint32_t prefix = 0u, mask = 0u;
    uint32_t need = static_cast<uint32_t>(kh);
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[lane] = 0u; hist[lane + 64] = 0u; hist[lane + 128] = 0u; hist[lane + 192] = 0u;
        wave_sync();
#pragma unroll
        for (int j = 0; j < kNplMax; ++j)
            if (j < npl && (u[j] & mask) == prefix) atomicAdd(&hist[(u[j] >> shift) & 255u], 1u);
        wave_sync();
        const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1];
        const uint32_t c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
        const uint32_t s = c0 + c1 + c2 + c3;
        uint32_t cb = wave_incl_scan_u32(s) - s;
        int found = -1;
        uint32_t fcb = 0u, fcnt = 0u;
        const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (found < 0 && cb < need && need <= cb + cs[j]) {
                found = 4 * lane + j;
                fcb = cb;
                fcnt = cs[j];
            }
            cb += cs[j];
        }
        const uint64_t bal = ballot(found >= 0);
        const int src = __ffsll(static_cast<unsigned long long>(bal)) - 1;
        const int d = __shfl(found, src, 64);
        fcb = __shfl(fcb, src, 64);
        fcnt = __shfl(fcnt, src, 64);
        prefix |= static_cast<uint32_t>(d) << shift;
        mask |= 0xffu << shift;
        need -= fcb;
        wave_sync();
        if (fcnt == need) break;
    }
    // Winners: below the prefix, or equal to it and among the first `need`
    // such elements in index order.
    uint32_t eq_base = 0u, sel_base = 0u;
    const uint64_t lt_mask = lanemask_lt();
#pragma unroll
    for (int j = 0; j < kNplMax; ++j) {
        if (j < npl) {
            const uint32_t x = u[j];
            const bool lt = (x & mask) < prefix;
            const bool eq = (x & mask) == prefix;
            const uint64_t eb = ballot(eq);
            const uint32_t er = eq_base + __popcll(eb & lt_mask);
            const bool sel = lt || (eq && er < need);
            const uint64_t sb = ballot(sel);
            const uint32_t pos = sel_base + __popcll(sb & lt_mask);
            if (sel) {
                out_e[pos] = __uint_as_float(x);
                out_i[pos] = j * 64 + lane;
            }
            eq_base += __popcll(eb);
            sel_base += __popcll(sb);
        }
    }
    wave_sync();
    uint64_t key[1];
    key[0] = (lane < kh) ? ((static_cast<uint64_t>(__float_as_uint(out_e[lane])) << 32) |
                            static_cast<uint32_t>(out_i[lane]))
                         : ~0ull;
    bitonic_sort<1>(key);
    if (lane < kh) {
        out_e[lane] = __uint_as_float(static_cast<uint32_t>(key[0] >> 32));
        out_i[lane] = static_cast<int>(key[0] & 0xffffffffu);
    }
    wave_sync();
}

// Product top-k of one (token, head) from the two sorted half lists.
template <int R>
__device__ void product_topk(const SweepArgs& a, const float* e1, const int* i1,
                             const float* e2, const int* i2, int32_t* idx_out, float* w_out) {
    const int lane = lane_id();
    uint64_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int c = r * 64 + lane;
        if (c < a.ncand) {
            const uint32_t ab = a.cand.ab[c];
            const int ia = static_cast<int>(ab >> 6), ib = static_cast<int>(ab & 63u);
            const float P = e1[ia] * e2[ib];
            const uint32_t slot = static_cast<uint32_t>(i1[ia] * a.n + i2[ib]);
            key[r] = (static_cast<uint64_t>(__float_as_uint(P)) << 32) | slot;
        } else {
            key[r] = ~0ull;
        }
    }
    bitonic_sort<R>(key);
    // the k best are elements 0..k-1, i.e. register 0 of lanes < k (k <= 64)
    const float P = __uint_as_float(static_cast<uint32_t>(key[0] >> 32));
    const float P0 = __shfl(P, 0, 64);
    const float ratio = (lane < a.k) ? (P0 / P) : 0.f;
    const float sum = wave_sum(ratio);
    if (lane < a.k) {
        idx_out[lane] = static_cast<int32_t>(key[0] & 0xffffffffu);
        w_out[lane] = ratio / sum;
    }
}

template <int STORE, int DHS>
__global__ __launch_bounds__(256) void k_sweep(SweepArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int n = a.n, H = a.H, dh = a.dh, kh = a.kh;
    const int ntiles = (a.Tc + kTileT - 1) / kTileT;
    const int estride = n + 4;  // padded LDS row (see bank mapping of the tile writes)
    float* et = reinterpret_cast<float*>(smem);                       // [16][estride]
    uint32_t* hist = reinterpret_cast<uint32_t*>(et + kTileT * estride);  // [4][256]
    float* sel_e = reinterpret_cast<float*>(hist + 4 * 256);           // [2][16][kh]
    int* sel_i = reinterpret_cast<int*>(sel_e + 2 * kTileT * kh);       // [2][16][kh]
    float* zrow = reinterpret_cast<float*>(sel_i + 2 * kTileT * kh);    // [16]

    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = static_cast<int>(lid % ntiles);
    const int bh = static_cast<int>(lid / ntiles);
    const int h = bh % H, b = bh / H;
    const int t0 = tile * kTileT;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int dq = 2 * dh;
    const int npl = (n + 63) >> 6;
    constexpr int ES = Store<STORE>::kBytes;

    for (int half = 0; half < 2; ++half) {
        const int bhh = (b * H + h) * 2 + half;
        const unsigned char* Kb = static_cast<const unsigned char*>(half ? a.K2 : a.K1) +
                                  static_cast<size_t>(b * H + h) * n * dh * ES;
        // query fragments of token t0 + r, this half
        Frag<STORE> A[DHS];
        const int tok = t0 + r;
        const bool tv = tok < a.Tc;
        const unsigned char* qrow = static_cast<const unsigned char*>(a.q) +
                                    (static_cast<size_t>(b) * a.q_bstride +
                                     static_cast<size_t>(tok) * H * dq + h * dq + half * dh) * ES;
        float qsq = 0.f;
#pragma unroll
        for (int s = 0; s < DHS; ++s) {
            if (tv) frag_load<STORE>(A[s], qrow + (32 * s + 8 * g) * ES);
            else frag_zero<STORE>(A[s]);
            qsq += frag_sumsq<STORE>(A[s]);
        }
        qsq += __shfl_xor(qsq, 16, 64);
        qsq += __shfl_xor(qsq, 32, 64);
        if (a.qn && wave == 0 && g == 0 && tv && (a.mode & (kSweepSelect | kSweepStats)))
            a.qn[static_cast<size_t>(bhh) * a.Tc + tok] = qsq;
        float qn_row[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) qn_row[i] = __shfl(qsq, 4 * g + i, 64);

        // distance tile: this wavefront takes key blocks wave, wave+4, ...
        const float* kn = a.knorm + static_cast<size_t>(bhh) * n;
        const int nkb = n >> 4;
        for (int kb = wave; kb < nkb; kb += 8) {
            const int kb2 = kb + 4;
            const bool two = kb2 < nkb;
            f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            const unsigned char* k0 = Kb + static_cast<size_t>(kb * 16 + r) * dh * ES;
            const unsigned char* k1 = Kb + static_cast<size_t>(kb2 * 16 + r) * dh * ES;
#pragma unroll
            for (int s = 0; s < DHS; ++s) {
                Frag<STORE> B0, B1;
                frag_load<STORE>(B0, k0 + (32 * s + 8 * g) * ES);
                if (two) frag_load<STORE>(B1, k1 + (32 * s + 8 * g) * ES);
                else frag_zero<STORE>(B1);
                mma(A[s], B0, acc0);
                mma(A[s], B1, acc1);
            }
            const float kn0 = kn[kb * 16 + r];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float d = qn_row[i] + kn0 - 2.f * acc0[i];
                et[(4 * g + i) * estride + kb * 16 + r] = a.eps + fmaxf(d, 0.f);
            }
            if (two) {
                const float kn1 = kn[kb2 * 16 + r];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d = qn_row[i] + kn1 - 2.f * acc1[i];
                    et[(4 * g + i) * estride + kb2 * 16 + r] = a.eps + fmaxf(d, 0.f);
                }
            }
        }
        __syncthreads();

        // per-token row work: wavefront w takes tokens 4w .. 4w+3 of the tile
        for (int tt = wave * 4; tt < wave * 4 + 4; ++tt) {
            const int tk = t0 + tt;
            if (tk >= a.Tc) break;
            uint32_t u[kNplMax];
#pragma unroll
            for (int j = 0; j < kNplMax; ++j) {
                const int i = j * 64 + lane;
                u[j] = (j < npl && i < n) ? __float_as_uint(et[tt * estride + i]) : 0x7f800000u;
            }
            if (a.mode & kSweepSelect) {
                wave_select(u, npl, kh, hist + wave * 256, sel_e + (half * kTileT + tt) * kh,
                            sel_i + (half * kTileT + tt) * kh);
            }
            if (a.mode & (kSweepStats | kSweepRowStat)) {
                float zs = 0.f, ms = 0.f;
                const float* lp = (a.mode & kSweepRowStat) ? a.lp + static_cast<size_t>(bhh) * n : nullptr;
#pragma unroll
                for (int j = 0; j < kNplMax; ++j) {
                    const int i = j * 64 + lane;
                    if (j < npl && i < n) {
                        const float inv = 1.f / __uint_as_float(u[j]);
                        zs += inv;
                        if (lp) ms = fmaf(inv, lp[i], ms);
                    }
                }
                zs = wave_sum(zs);
                if (lane == 0) zrow[tt] = zs;
                if (a.mode & kSweepRowStat) {
                    ms = wave_sum(ms);
                    if (lane == 0) {
                        a.Z[static_cast<size_t>(bhh) * a.Tc + tk] = zs;
                        a.m[static_cast<size_t>(bhh) * a.Tc + tk] = ms / zs;
                    }
                }
            }
        }
        __syncthreads();

        if (a.mode & kSweepStats) {
            const int nvalid = min(kTileT, a.Tc - t0);
            float* part = a.part + (static_cast<size_t>(bhh) * ntiles + tile) * n;
            for (int i = threadIdx.x; i < n; i += 256) {
                float s = 0.f;
                for (int tt = 0; tt < nvalid; ++tt) s += (1.f / et[tt * estride + i]) / zrow[tt];
                part[i] = s;
            }
        }
        __syncthreads();
    }

    if (a.mode & kSweepSelect) {
        for (int tt = wave * 4; tt < wave * 4 + 4; ++tt) {
            const int tk = t0 + tt;
            if (tk >= a.Tc) break;
            const size_t o = static_cast<size_t>(b) * a.iw_bstride + (static_cast<size_t>(tk) * H + h) * a.k;
            const float* e1 = sel_e + (0 * kTileT + tt) * kh;
            const int* i1 = sel_i + (0 * kTileT + tt) * kh;
            const float* e2 = sel_e + (1 * kTileT + tt) * kh;
            const int* i2 = sel_i + (1 * kTileT + tt) * kh;
            if (a.ncand <= 64) product_topk<1>(a, e1, i1, e2, i2, a.idx + o, a.w + o);
            else if (a.ncand <= 128) product_topk<2>(a, e1, i1, e2, i2, a.idx + o, a.w + o);
            else product_topk<4>(a, e1, i1, e2, i2, a.idx + o, a.w + o);
        }
    }
}

template <int STORE, int DHS>
hipError_t launch_sweep_t(const SweepArgs& a, hipStream_t s) {
    const int ntiles = (a.Tc + kTileT - 1) / kTileT;
    const size_t lds = (static_cast<size_t>(kTileT) * (a.n + 4) + 4 * 256 + 4 * kTileT * a.kh + kTileT) * 4;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_sweep<STORE, DHS>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const unsigned grid = static_cast<unsigned>(a.B) * a.H * ntiles;
    hipLaunchKernelGGL((k_sweep<STORE, DHS>), dim3(grid), dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sweep(const SweepArgs& a, int store, hipStream_t s) {
    const int dhs = a.dh / 32;
    if (store == kBF16) {
        switch (dhs) {
            case 1: return launch_sweep_t<kBF16, 1>(a, s);
            case 2: return launch_sweep_t<kBF16, 2>(a, s);
            case 4: return launch_sweep_t<kBF16, 4>(a, s);
            case 8: return launch_sweep_t<kBF16, 8>(a, s);
        }
    } else {
        switch (dhs) {
            case 1: return launch_sweep_t<kF32, 1>(a, s);
            case 2: return launch_sweep_t<kF32, 2>(a, s);
            case 4: return launch_sweep_t<kF32, 4>(a, s);
            case 8: return launch_sweep_t<kF32, 8>(a, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace fwpkm
