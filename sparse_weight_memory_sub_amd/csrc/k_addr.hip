// k_addr.hip -- addressing (anti-collapse) step on the sub-key codebooks.
//
// "Fast-weight Product Key Memory", rainbus digest step 5 and paperlayer.ai
// 3.4: the keys take one gradient step on L = -H(pbar_1) - H(pbar_2), the
// negative entropies of the chunk's marginal sub-key usage.  With
// e_ti = eps + ||q_t - K_i||^2, p_ti = (1/e_ti) / Z_t (softmax of the IDW
// score s = -log e over all n sub-keys), pbar_i = mean_t p_ti and
// m_t = sum_i p_ti log pbar_i, the chain rule through the softmax and the
// score gives
//   dL/dK_i = sum_t a_ti (q_t - K_i),   a_ti = 2 (log pbar_i - m_t) / (Tc Z_t e_ti^2).
//
// k_kgrad: one workgroup per 64 sub-keys of one (sequence, head, half); each
// wavefront owns 16 keys and walks the chunk's tokens in blocks of 32:
//  1. recompute the 32x16 distance tile on the matrix cores (same fragments
//     and order as the scoring sweep, so the values are bitwise the same);
//  2. form a_ti for its keys;
//  3. accumulate sum_t a_ti q_t on the matrix cores (keys x tokens times
//     tokens x d_h; for bf16 storage a_ti is split into a bf16 high part and
//     a bf16 low part, two MFMAs, about 16 bits of a_ti).
// Then K_i <- K_i - lr (sum_t a_ti q_t - (sum_t a_ti) K_i), rounded to the
// storage type, and ||K_i||^2 of the stored key is written for the next
// chunk's scoring.  Every key is read and written by one wavefront only.
#include "mfma_frag.h"

namespace fwpkm {

namespace {

// log pbar_i from the per-tile partial sums, tiles added in order.
__global__ __launch_bounds__(256) void k_pbar(PbarArgs a) {
    const int bhh = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= a.n) return;
    const float* part = a.part + static_cast<size_t>(bhh) * a.ntiles * a.n + i;
    float s = 0.f;
    for (int t = 0; t < a.ntiles; ++t) s += part[static_cast<size_t>(t) * a.n];
    a.lp[static_cast<size_t>(bhh) * a.n + i] = logf(s / static_cast<float>(a.Tc));
}

// ||K_i||^2 for every sub-key.  Sixteen lanes per key; lane r adds the
// squares of columns r, r+16, r+32, ... in order, then the sixteen partial
// sums are combined by an xor butterfly.  This is the same order as the norm
// k_kgrad writes after its step, so a chunk scores with the same key norms
// whether the previous chunk's step ran in the same call or not.
template <int STORE>
__global__ __launch_bounds__(256) void k_knorm(KnormArgs a) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15;
    const int64_t key = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);  // over B*H*2*n
    const int64_t total = static_cast<int64_t>(a.B) * a.H * 2 * a.n;
    const bool valid = key < total;
    float x = 0.f;
    if (valid) {
        const int i = static_cast<int>(key % a.n);
        const int64_t bhh = key / a.n;
        const int half = static_cast<int>(bhh % 2);
        const int64_t bh = bhh / 2;
        const void* K = half ? a.K2 : a.K1;
        const size_t base = (static_cast<size_t>(bh) * a.n + i) * a.dh;
        for (int c = 0; c < a.dh / 16; ++c) {
            const float v = ld_elem<STORE>(K, base + c * 16 + r);
            x = fmaf(v, v, x);
        }
    }
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    if (valid && r == 0) a.knorm[key] = x;
}

__device__ __forceinline__ uint32_t bf16_bits(float x) { return f32_to_bf16(x); }

// token of element j of lane group g in the 32-token block: the first four
// from the 16-token sub-tile 0, the last four from sub-tile 1, matching the
// row layout of the MFMA distance tiles.
__device__ __forceinline__ int tok_of(int g, int j) { return (j < 4) ? (4 * g + j) : (16 + 4 * g + j - 4); }

template <int STORE, int DHS>
__global__ __launch_bounds__(256) void k_kgrad(KgradArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int PAD = (STORE == kBF16) ? 8 : 4;  // row padding in elements (LDS banks)
    const int dh = a.dh, n = a.n, H = a.H;
    const int qstride = dh + PAD;
    unsigned char* qs = smem;                                            // [32][qstride]
    float* tq = reinterpret_cast<float*>(smem + 32 * qstride * ES);     // qn, Z, m: [3][32]

    const int nkb = (n + 63) / 64;
    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int kb = static_cast<int>(lid % nkb);
    int rest = static_cast<int>(lid / nkb);
    const int half = rest % 2;
    rest /= 2;
    const int h = rest % H, b = rest / H;
    const int bhh = (b * H + h) * 2 + half;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int key0 = kb * 64 + wave * 16;
    const bool active = key0 < n;
    const int key = key0 + r;
    unsigned char* Kb = static_cast<unsigned char*>(half ? a.K2 : a.K1) + static_cast<size_t>(b * H + h) * n * dh * ES;
    const int dq = 2 * dh;

    Frag<STORE> Bk[DHS];
    float kn = 0.f, lpv = 0.f;
    if (active) {
        load_row_frags<STORE, DHS>(Bk, Kb + static_cast<size_t>(key) * dh * ES, g);
        kn = a.knorm[static_cast<size_t>(bhh) * n + key];
        lpv = a.lp[static_cast<size_t>(bhh) * n + key];
    }
    constexpr int NCT = DHS * 2;  // 16-wide column tiles of d_h
    f32x4_t gacc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) gacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float colsum = 0.f;
    const float inv_tc2 = 2.f / static_cast<float>(a.Tc);

    // key blocks of one (sequence, head, half) run side by side and read the
    // same query rows: start each at a different token block (fixed order per
    // block, so the sums stay reproducible)
    const int nblk = (a.Tc + 31) / 32;
    for (int bi = 0; bi < nblk; ++bi) {
        const int tb = ((bi + kb) % nblk) * 32;
        __syncthreads();
        // stage the query halves of tokens tb .. tb+31 (zeros past Tc)
        const int chunks = dh / 8;  // 8-element pieces per row
        for (int c = threadIdx.x; c < 32 * chunks; c += 256) {
            const int row = c / chunks, col = (c % chunks) * 8;
            const int t = tb + row;
            unsigned char* dst = qs + (static_cast<size_t>(row) * qstride + col) * ES;
            if (t < a.Tc) {
                const unsigned char* src = static_cast<const unsigned char*>(a.q) +
                    (static_cast<size_t>(b) * a.q_bstride + static_cast<size_t>(t) * H * dq + h * dq + half * dh + col) * ES;
                if constexpr (STORE == kBF16) {
                    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
                } else {
                    reinterpret_cast<float4*>(dst)[0] = reinterpret_cast<const float4*>(src)[0];
                    reinterpret_cast<float4*>(dst)[1] = reinterpret_cast<const float4*>(src)[1];
                }
            } else {
                if constexpr (STORE == kBF16) {
                    *reinterpret_cast<uint4*>(dst) = make_uint4(0u, 0u, 0u, 0u);
                } else {
                    reinterpret_cast<float4*>(dst)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
                    reinterpret_cast<float4*>(dst)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
        if (threadIdx.x < 96) {
            const int which = threadIdx.x / 32, row = threadIdx.x % 32;
            const int t = tb + row;
            const float* src = which == 0 ? a.qn : (which == 1 ? a.Z : a.m);
            float x = (t < a.Tc) ? src[static_cast<size_t>(bhh) * a.Tc + t] : 1.f;
            if (which == 1) x = __builtin_amdgcn_rcpf(x);  // stored as 1/Z
            tq[which * 32 + row] = x;
        }
        __syncthreads();
        if (!active) continue;

        float av[8];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            Frag<STORE> A[DHS];
            load_row_frags<STORE, DHS>(A, qs + static_cast<size_t>(sub * 16 + r) * qstride * ES, g);
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DHS; ++s) mma(A[s], Bk[s], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = sub * 16 + 4 * g + i;
                const float d = tq[row] + kn - 2.f * acc[i];
                const float ie = __builtin_amdgcn_rcpf(a.eps + fmaxf(d, 0.f));
                const float val = (tb + row < a.Tc) ? inv_tc2 * (lpv - tq[64 + row]) * tq[32 + row] * ie * ie : 0.f;
                av[sub * 4 + i] = val;
                colsum += val;
            }
        }
        // sum_t a_ti q_t: keys x tokens (A) times tokens x d_h (B)
        Frag<kBF16> Ahi, Alo;
        if constexpr (STORE == kBF16) {
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                hi[j] = pack_bf16x2(av[2 * j], av[2 * j + 1]);
                lo[j] = pack_bf16x2(av[2 * j] - __uint_as_float(hi[j] << 16),
                                    av[2 * j + 1] - __uint_as_float(hi[j] & 0xffff0000u));
            }
            Ahi.v = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
            Alo.v = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
        }
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            const int col = c * 16 + r;
            if constexpr (STORE == kBF16) {
                const uint16_t* qb = reinterpret_cast<const uint16_t*>(qs);
                uint32_t bq[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) bq[j] = qb[tok_of(g, j) * qstride + col];
                Frag<kBF16> B;
                B.v = u32x4_t{bq[0] | (bq[1] << 16), bq[2] | (bq[3] << 16), bq[4] | (bq[5] << 16), bq[6] | (bq[7] << 16)};
                mma(Ahi, B, gacc[c]);
                mma(Alo, B, gacc[c]);
            } else {
                const float* qf = reinterpret_cast<const float*>(qs);
                Frag<kF32> B, A;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    B.v[j] = qf[tok_of(g, j) * qstride + col];
                    A.v[j] = av[j];
                }
                mma(A, B, gacc[c]);
            }
        }
    }
    if (!active) return;

    // colsum over the four lane groups: lanes with the same r hold the same key
    colsum += __shfl_xor(colsum, 16, 64);
    colsum += __shfl_xor(colsum, 32, 64);
    float cs[4], ksq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        cs[i] = __shfl(colsum, 4 * g + i, 64);
        ksq[i] = 0.f;
    }
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        const int col = c * 16 + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = key0 + 4 * g + i;
            const size_t off = static_cast<size_t>(k) * dh + col;
            const float kv = ld_elem<STORE>(Kb, off);
            const float grad = gacc[c][i] - cs[i] * kv;
            float kn2 = kv - a.lr * grad;
            if constexpr (STORE == kBF16) kn2 = bf16_to_f32(f32_to_bf16(kn2));
            st_elem<STORE>(Kb, off, kn2);
            ksq[i] = fmaf(kn2, kn2, ksq[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x = ksq[i];
        x += __shfl_xor(x, 1, 64);
        x += __shfl_xor(x, 2, 64);
        x += __shfl_xor(x, 4, 64);
        x += __shfl_xor(x, 8, 64);
        if (r == 0) a.knorm[static_cast<size_t>(bhh) * n + key0 + 4 * g + i] = x;
    }
}

template <int STORE, int DHS>
hipError_t kgrad_t(const KgradArgs& a, hipStream_t s) {
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int PAD = (STORE == kBF16) ? 8 : 4;
    const size_t lds = static_cast<size_t>(32) * (a.dh + PAD) * ES + 3 * 32 * 4;
    const int nkb = (a.n + 63) / 64;
    const unsigned grid = static_cast<unsigned>(a.B) * a.H * 2 * nkb;
    hipLaunchKernelGGL((k_kgrad<STORE, DHS>), dim3(grid), dim3(256), lds, s, a);
    return hipGetLastError();
}

template <int STORE>
hipError_t kgrad_s(const KgradArgs& a, hipStream_t s) {
    switch (a.dh / 32) {
        case 1: return kgrad_t<STORE, 1>(a, s);
        case 2: return kgrad_t<STORE, 2>(a, s);
        case 4: return kgrad_t<STORE, 4>(a, s);
        case 8: return kgrad_t<STORE, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_pbar(const PbarArgs& a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((a.n + 255) / 256), static_cast<unsigned>(a.B * a.H * 2));
    hipLaunchKernelGGL(k_pbar, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_knorm(const KnormArgs& a, int store, hipStream_t s) {
    const int64_t keys = static_cast<int64_t>(a.B) * a.H * 2 * a.n;
    const unsigned grid = static_cast<unsigned>((keys + 15) / 16);
    if (store == kBF16) hipLaunchKernelGGL(k_knorm<kBF16>, dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_knorm<kF32>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_kgrad(const KgradArgs& a, int store, hipStream_t s) {
    return store == kBF16 ? kgrad_s<kBF16>(a, s) : kgrad_s<kF32>(a, s);
}

}  // namespace fwpkm
