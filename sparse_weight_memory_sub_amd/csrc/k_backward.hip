// k_backward.hip -- gradient of the retrieval output with respect to the
// query, the residual-path value and the gate.
//
// The forward ("Fast-weight Product Key Memory": rainbus digest steps 2-3,
// paperlayer.ai 2.2, 3.2, A.2) is, per token and head, the pair scores
// S_j = -log(eps + d1_j) - log(eps + d2_j) of the k selected slots, weights
// w = softmax(S), v_hat = (1/H) sum_h sum_j w_j V[slot_j] and
// o = g v_hat + (1 - g) v.  With the selection and the fast-weight state held
// fixed, for an upstream gradient G = dL/do:
//   dL/dg = G . (v_hat - v),  dL/dv = (1 - g) G,
//   a_j = (g/H) G . V[slot_j],  dL/dS_j = w_j (a_j - sum_l w_l a_l),
//   dL/dq_half = sum_j dL/dS_j * (-2) (q_half - K_half[sub_j]) / (eps + d_j),
// or with dot-product scores (S_j = q1 . K1[a_j] + q2 . K2[b_j])
//   dL/dq_half = sum_j dL/dS_j K_half[sub_j].
// The distances are recomputed by direct differences.
//
// One wavefront per token.  The value rows are read as in the gather (lane l
// owns d_v elements [l*EPL, (l+1)*EPL)), eight at a time, their eight dot
// products reduced together.  For the query part the wavefront splits into
// four 16-lane groups, each taking one selected sub-key row at a time over
// d_h.  Slot ids outside [0, N) are skipped.
#include "rows.h"

namespace fwpkm {

namespace {

// Eight partial sums per lane -> their wavefront totals: a butterfly that
// halves the set at each of the first three exchanges.  On return lane L
// holds the total of value (L >> 3).
__device__ __forceinline__ float reduce8(const float (&d)[8]) {
    const int lane = __lane_id();
    float x4[4], x2[2];
    const bool h5 = (lane & 32) != 0, h4 = (lane & 16) != 0, h3 = (lane & 8) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float keep = h5 ? d[i + 4] : d[i], give = h5 ? d[i] : d[i + 4];
        x4[i] = keep + xor_lane(give, 32);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float keep = h4 ? x4[i + 2] : x4[i], give = h4 ? x4[i] : x4[i + 2];
        x2[i] = keep + xor_lane(give, 16);
    }
    float x = (h3 ? x2[1] : x2[0]) + xor_lane(h3 ? x2[0] : x2[1], 8);
    x += xor_lane(x, 4);
    x += xor_lane(x, 2);
    x += xor_lane(x, 1);
    return x;
}

// E consecutive storage elements from element offset off as floats.
template <int STORE, int E>
__device__ __forceinline__ void ld_seg(const void* base, size_t off, float (&x)[E]) {
    if constexpr (E <= 8) {
        ldrow<STORE, E>(base, off, x);
    } else {
        float y[8];
#pragma unroll
        for (int c = 0; c < E / 8; ++c) {
            ldrow<STORE, 8>(base, off + 8 * c, y);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[8 * c + i] = y[i];
        }
    }
}

template <int STORE, int EPL, int DHS, bool DOT>
__global__ __launch_bounds__(256) void k_backward(BackwardArgs a) {
    constexpr int DH = 32 * DHS;
    constexpr int EPQ = DH / 16;  // elements of a half row per lane of a 16-lane group
    __shared__ int32_t lsl[4][256];
    __shared__ float lds_a[4][256];
    __shared__ float lds_ds[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (tok >= static_cast<int64_t>(a.B) * a.T) return;
    const int b = static_cast<int>(tok / a.T), t = static_cast<int>(tok % a.T);
    const int H = a.H, k = a.k, HK = H * k, dv = a.dv, n = a.n;
    const size_t iwo = static_cast<size_t>(b) * a.iw_bstride + static_cast<size_t>(t) * HK;
    const size_t vo = static_cast<size_t>(b) * a.v_bstride + static_cast<size_t>(t) * dv;
    const size_t go = static_cast<size_t>(b) * a.g_bstride + t;
    const size_t col = static_cast<size_t>(lane) * EPL;

    // entry e = h*k + j: slot and weight in lane e % 64 of register e / 64
    int32_t sl[4];
    float wt[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = r * 64 + lane;
        sl[r] = (e < HK) ? a.idx[iwo + e] : 0;
        wt[r] = (e < HK) ? a.w[iwo + e] : 0.f;
        if (e < HK) lsl[wave][e] = sl[r];
    }
    float G[EPL];
    ldrow<kF32, EPL>(a.dO, vo + col, G);
    const float gt = a.g[go];
    const float gh = gt / static_cast<float>(H);
    const size_t vb = static_cast<size_t>(b) * static_cast<size_t>(a.N) * dv;

    // value part: v_hat and a_e = (g/H) G . V[slot_e], eight rows at a time
    float vh[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) vh[i] = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int cnt = min(64, HK - r * 64);
        if (cnt <= 0) break;
        for (int j0 = 0; j0 < cnt; j0 += 8) {
            // the eight rows' loads all in flight before their use; an id
            // outside [0, N) reads row 0 in its place and contributes nothing
            float dot[8], x[8][EPL], ww[8];
            bool ok[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s = (j0 + u < cnt) ? __builtin_amdgcn_readlane(sl[r], j0 + u) : -1;
                ok[u] = s >= 0 && s < a.N;
                ww[u] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt[r]), min(j0 + u, 63)));
                ldrow<STORE, EPL, true>(a.V, vb + static_cast<size_t>(ok[u] ? s : 0) * dv + col, x[u]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                dot[u] = 0.f;
                if (ok[u]) {
#pragma unroll
                    for (int i = 0; i < EPL; ++i) {
                        vh[i] = fmaf(ww[u], x[u][i], vh[i]);
                        dot[u] = fmaf(G[i], x[u][i], dot[u]);
                    }
                }
            }
            const float tot = reduce8(dot);
            const int u = lane >> 3;
            if ((lane & 7) == 0 && j0 + u < cnt) lds_a[wave][r * 64 + j0 + u] = gh * tot;
        }
    }
    {
        float vt[EPL];
        ldrow<STORE, EPL>(a.v, vo + col, vt);
        float p = 0.f, dvv[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            p = fmaf(G[i], vh[i] / static_cast<float>(H) - vt[i], p);
            dvv[i] = (1.f - gt) * G[i];
        }
        const float dg = wave_sum(p);
        if (lane == 0) a.dg[go] = dg;
        stf<EPL>(a.dv_out + vo + col, dvv);
    }
    wave_sync();

    // softmax backward per head: dS_e = w_e (a_e - sum over the head of w a)
    float ar[4], wa[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int e = r * 64 + lane;
        ar[r] = (e < HK) ? lds_a[wave][e] : 0.f;
        wa[r] = wt[r] * ar[r];
    }
    for (int h = 0; h < H; ++h) {
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = r * 64 + lane;
            if (e >= h * k && e < (h + 1) * k) part += wa[r];
        }
        const float A = wave_sum(part);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = r * 64 + lane;
            if (e >= h * k && e < (h + 1) * k) lds_ds[wave][e] = wt[r] * (ar[r] - A);
        }
    }
    wave_sync();

    // query part: four 16-lane groups take one selected slot each; lane gl
    // of a group owns elements [gl*EPQ, +EPQ) of the half row
    const int grp = lane >> 4, gl = lane & 15;
    for (int h = 0; h < H; ++h) {
        for (int hf = 0; hf < 2; ++hf) {
            const size_t qoff = static_cast<size_t>(b) * a.q_bstride + (static_cast<size_t>(t) * H + h) * (2 * DH) +
                                static_cast<size_t>(hf) * DH + gl * EPQ;
            const void* Kh = hf ? a.K2 : a.K1;
            const size_t kb = static_cast<size_t>(b * H + h) * n * DH + gl * EPQ;
            float qv[EPQ], acc[EPQ];
            ld_seg<STORE, EPQ>(a.q, qoff, qv);
#pragma unroll
            for (int i = 0; i < EPQ; ++i) acc[i] = 0.f;
            // a group's slots j = grp, grp + 4, ... in order, KQ sub-key rows
            // requested before the first is used
            constexpr int KQ = 4;
            for (int j0 = 0; j0 < k; j0 += 4 * KQ) {
                float kx[KQ][EPQ];
                int e[KQ];
                bool ok[KQ];
#pragma unroll
                for (int c = 0; c < KQ; ++c) {
                    const int j = j0 + 4 * c + grp;
                    e[c] = h * k + j;
                    const int32_t slot = (j < k) ? lsl[wave][e[c]] : -1;
                    ok[c] = slot >= 0 && slot < a.N;
                    const int sub = ok[c] ? (hf ? slot % n : slot / n) : 0;
                    ld_seg<STORE, EPQ>(Kh, kb + static_cast<size_t>(sub) * DH, kx[c]);
                }
#pragma unroll
                for (int c = 0; c < KQ; ++c) {
                    if constexpr (DOT) {
                        // dS/dq_half = K_half[sub]
                        const float coef = ok[c] ? lds_ds[wave][e[c]] : 0.f;
#pragma unroll
                        for (int i = 0; i < EPQ; ++i) acc[i] = fmaf(coef, kx[c][i], acc[i]);
                    } else {
                        float diff[EPQ], part = 0.f;
#pragma unroll
                        for (int i = 0; i < EPQ; ++i) {
                            diff[i] = qv[i] - kx[c][i];
                            part = fmaf(diff[i], diff[i], part);
                        }
                        part += xor_lane(part, 1);
                        part += xor_lane(part, 2);
                        part += xor_lane(part, 4);
                        part += xor_lane(part, 8);
                        const float coef = ok[c] ? lds_ds[wave][e[c]] * (-2.f) / (a.eps + part) : 0.f;
#pragma unroll
                        for (int i = 0; i < EPQ; ++i) acc[i] = fmaf(coef, diff[i], acc[i]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < EPQ; ++i) {
                acc[i] += xor_lane(acc[i], 16);
                acc[i] += xor_lane(acc[i], 32);
            }
            if (grp == 0) {
                float* dq = a.dq + qoff;
                if constexpr (EPQ % 4 == 0) {
#pragma unroll
                    for (int i = 0; i < EPQ; i += 4)
                        *reinterpret_cast<float4*>(dq + i) = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
                } else {
#pragma unroll
                    for (int i = 0; i < EPQ; ++i) dq[i] = acc[i];
                }
            }
        }
    }
}

template <int STORE, int EPL, int DHS>
hipError_t backward_k(const BackwardArgs& a, unsigned grid, hipStream_t s) {
    if (a.dot) hipLaunchKernelGGL((k_backward<STORE, EPL, DHS, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_backward<STORE, EPL, DHS, false>), dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int STORE, int EPL>
hipError_t backward_d(const BackwardArgs& a, unsigned grid, hipStream_t s) {
    switch (a.dh / 32) {
        case 1: return backward_k<STORE, EPL, 1>(a, grid, s);
        case 2: return backward_k<STORE, EPL, 2>(a, grid, s);
        case 4: return backward_k<STORE, EPL, 4>(a, grid, s);
        case 8: return backward_k<STORE, EPL, 8>(a, grid, s);
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int STORE>
hipError_t backward_s(const BackwardArgs& a, hipStream_t s) {
    const int64_t toks = static_cast<int64_t>(a.B) * a.T;
    const unsigned grid = static_cast<unsigned>((toks + 3) / 4);
    switch (a.dv / 64) {
        case 1: return backward_d<STORE, 1>(a, grid, s);
        case 2: return backward_d<STORE, 2>(a, grid, s);
        case 4: return backward_d<STORE, 4>(a, grid, s);
        case 8: return backward_d<STORE, 8>(a, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, int store, hipStream_t s) {
    if (a.B <= 0 || a.T <= 0) return hipSuccess;
    return store == kBF16 ? backward_s<kBF16>(a, s) : backward_s<kF32>(a, s);
}

}  // namespace fwpkm
