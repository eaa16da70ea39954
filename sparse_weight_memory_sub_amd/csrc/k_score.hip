// k_score.hip -- sub-key scoring of a chunk against both half codebooks.
//
// Scoring ("Fast-weight Product Key Memory": paperlayer.ai 2.2 and A.2,
// rainbus digest step 2): the query is split into halves and each half is
// compared with every sub-key of its codebook by squared Euclidean distance,
// computed as ||q||^2 + ||K_i||^2 - 2 q.K_i on the matrix cores; the score
// is s = -log(eps + d).  Statistics of the addressing step (digest step 5,
// paperlayer.ai 3.4) use p_ti = (1/e_ti) / Z_t, e = eps + d, Z_t = sum_i 1/e_ti.
//
// k_score streams the codebook through LDS like a GEMM: a workgroup owns a
// tile of 64, 128 or 256 tokens of one (sequence, head, half) -- 16 per
// wavefront, the MFMA rows -- and walks the sub-keys in blocks of kKB,
// double-buffered and copied by direct global-to-LDS loads, so every sub-key
// row is read from L2 once per tile.  The tile is the widest that still gives
// every compute unit a workgroup: wide tiles share each staged block (and its
// barrier) among more tokens, narrow ones spread a small batch over more CUs.
// The accumulators start at ||K_i||^2 and the query is scaled by -2, so the
// MFMAs leave ||K_i||^2 - 2 q.K_i, summed at the small magnitude
// of the dot products; ||q||^2 + eps is added once at the end (one rounding
// at the scale of ||q||^2, which may dwarf the spread of the distances).  Nothing
// of the distance matrix is stored; each mode (a template argument) reduces
// it in registers:
//
//  kScoreSelect   pass 1: for each lane the MK smallest e of the sub-keys it
//                 sees; tau_t = k'-th smallest of those 16*MK values is an
//                 upper bound of the k'-th smallest e of the row (at least
//                 k' values are <= tau_t).  Pass 2 recomputes the tile and
//                 appends every (e, sub-key) with e <= tau_t to the token's
//                 candidate list in the workspace (positions from a ballot
//                 of the token row's lanes; k_select sorts the list).
//  kScoreStats    pass 1 also sums Z_t = sum_i 1/e_ti (written out); pass 2
//                 forms the per-tile partial sums over tokens of p_ti,
//                 the pieces of the chunk's marginal usage pbar.
//  kScoreRowStat  one pass: m_t = sum_i p_ti log pbar_i, with Z_t from the
//                 stats pass of the same chunk.
//
// k_select: one wavefront per (token, head): sorts each half's candidates
// by (e, sub-key) for the top-k' (ties to the lower sub-key index), then the
// top-k of the product candidates by P = e1*e2 (ties to the lower slot id
// i*n + j) and the weights (1/P)/sum(1/P) = softmax of s1 + s2.  A token
// whose candidate list overflowed recomputes its distances exactly and
// selects by radix select.
#include "gather.h"
#include "mfma_frag.h"

namespace fwpkm {

namespace {

// sub-keys per LDS block: 32 bf16 or 16 fp32 rows (at most 16 KiB for d_h <= 256);
// 64 bf16 rows (32 KiB) for the widest tiles, which hold a compute unit
// alone and meet at half as many barriers
template <int STORE, int NW> constexpr int kKB = (STORE == kBF16) ? (NW >= 16 ? 64 : 32) : 16;
constexpr int kNplMax = 16;    // sub-keys per lane in a row: n <= 1024

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    const uint32_t lo = xor_lane(static_cast<uint32_t>(x), m);
    const uint32_t hi = xor_lane(static_cast<uint32_t>(x >> 32), m);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Ascending bitonic sort of R*W keys held by groups of W lanes (W = 64 or
// 16): element p = r*W + (lane % W) of each group.
template <int R, int W, typename K>
__device__ __forceinline__ void bitonic_sort(K (&x)[R]) {
    const int ln = lane_id() & (W - 1);
#pragma unroll
    for (int size = 2; size <= W * R; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= W) {
                const int rs = stride / W;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if ((r & rs) == 0) {
                        const int r2 = r | rs;
                        const int p = r * W + ln;
                        const bool up = (p & size) == 0;
                        const K a = x[r], b = x[r2];
                        // swap if out of order for the direction: one compare
                        // (equal keys swap or not: the same values either way)
                        const bool sw = (a > b) == up;
                        x[r] = sw ? b : a;
                        x[r2] = sw ? a : b;
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    K y;
                    if constexpr (sizeof(K) == 8) y = shfl_xor_u64(x[r], stride);
                    else y = xor_lane(x[r], stride);
                    const int p = r * W + ln;
                    const bool up = (p & size) == 0;
                    const bool lower = (ln & stride) == 0;
                    // keep x when it is the one this lane wants (the smaller
                    // for the lower lane of an ascending pair): one compare
                    x[r] = ((x[r] < y) == (lower == up)) ? x[r] : y;
                }
            }
        }
    }
}

// Ascending bitonic sort of L independent 64-element lists, list l in x[l]
// (element = lane).  The lists go through the network side by side, so the
// lane exchanges of one list fill the latency of the other's.
template <int L>
__device__ __forceinline__ void bitonic_sort_lists(uint64_t (&x)[L]) {
    const int ln = lane_id();
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const bool up = (ln & size) == 0;
            const bool lower = (ln & stride) == 0;
#pragma unroll
            for (int l = 0; l < L; ++l) {
                const uint64_t y = shfl_xor_u64(x[l], stride);
                x[l] = ((x[l] < y) == (lower == up)) ? x[l] : y;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_score
// ---------------------------------------------------------------------------

// One sweep of a tile of 16*NW*TG tokens of one (sequence, head, half)
// against all n sub-keys of that half.  Each wavefront owns TG groups of 16
// tokens (the MFMA rows); every sub-key fragment it reads from LDS feeds the
// MFMAs of all TG groups, so two groups halve the LDS reads per distance.
// Each group's arithmetic is that of a wavefront of its own (the same MFMA
// order per accumulator; per-token and per-column sums over the groups in
// token order).  The launches use one group per wavefront: two (170
// registers, two wavefronts per SIMD) made the 2^20-slot sweep slower,
// 128 -> 170 us.  MODE is a combination of kScoreSelect, kScoreStats and
// kScoreRowStat (the latter alone).
template <int STORE, int DHS, int MK, int MODE, int NW, int TG, bool DOT>
__global__ __launch_bounds__(64 * NW) void k_score(ScoreArgs a) {
    static_assert(TG >= 1 && TG <= 4, "a workgroup's counters are zeroed by one thread per token");
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int KB = kKB<STORE, NW>;
    constexpr int CPR = 32 * DHS * ES / 16;
    constexpr int BLK_BYTES = KB * CPR * 16;
    constexpr bool SEL = (MODE & kScoreSelect) != 0;
    constexpr bool STATS = (MODE & kScoreStats) != 0;
    constexpr bool ROW = (MODE & kScoreRowStat) != 0;
    constexpr int NPASS = (SEL || STATS) ? 2 : 1;
    constexpr int NG = NW * TG;  // 16-token groups of the workgroup
    constexpr int TT = 16 * NG;  // tokens of the workgroup
    extern __shared__ __align__(16) unsigned char smem[];
    unsigned char* kbuf = smem;                                            // [2][BLK_BYTES]
    float* kns = reinterpret_cast<float*>(smem + 2 * BLK_BYTES);           // [n]  ||K_i||^2
    float* colbuf = kns + a.n;                                             // [2][NG][KB] (stats)
    float* lps = colbuf + (STATS ? 2 * NG * KB : 0);                       // [n]  log pbar (row statistic)

    const int n = a.n, H = a.H, Tc = a.Tc;
    const int ntiles = (Tc + TT - 1) / TT;
    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = static_cast<int>(lid % ntiles);
    const int bhh = static_cast<int>(lid / ntiles);  // (b*H + h)*2 + half
    const int half = bhh & 1, bh = bhh >> 1;
    const int h = bh % H, b = bh / H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int tw0 = tile * TT + wave * 16 * TG;  // first token of this wavefront; group j from tw0 + 16 j
    const int nblk = (n + KB - 1) / KB;
    const unsigned char* Kg = static_cast<const unsigned char*>(half ? a.K2 : a.K1) +
                              static_cast<size_t>(bh) * n * (32 * DHS) * ES;
    const size_t rowbase = static_cast<size_t>(bhh) * Tc;
    for (int i = threadIdx.x; i < n; i += 64 * NW) kns[i] = a.knorm[static_cast<size_t>(bhh) * n + i];

    // query fragments of token tw0 + 16 j + r (zero past the chunk), then -2 q
    Frag<STORE> A[TG][DHS];
    float qe[TG][4];
    bool rv[TG][4];
    const int eps_bits = __float_as_int(a.eps);
#pragma unroll
    for (int j = 0; j < TG; ++j) {
        const int tok = tw0 + 16 * j + r;
        const bool tv = tok < Tc;
        const unsigned char* qrow = static_cast<const unsigned char*>(a.q) +
            (static_cast<size_t>(b) * a.q_bstride + static_cast<size_t>(tv ? tok : 0) * H * (64 * DHS) +
             h * (64 * DHS) + half * (32 * DHS)) * ES;
        load_row_frags<STORE, DHS>(A[j], qrow, g);
        float qsq = 0.f;
#pragma unroll
        for (int s = 0; s < DHS; ++s) {
            if (!tv) frag_zero<STORE>(A[j][s]);
            qsq += frag_sumsq<STORE>(A[j][s]);
            if constexpr (!DOT) frag_scale_m2(A[j][s]);  // dot scores use q itself
            // the scaled fragment is formed here: left free, the compiler
            // keeps the unpacked elements of ||q||^2 live until the loop to
            // scale them there, and the kernel's peak register count with
            // them (the 2^20-slot sweep: 112 -> 104)
            if constexpr (STORE == kBF16) asm volatile("" : "+v"(A[j][s].v));
        }
        qsq += xor_lane(qsq, 16);
        qsq += xor_lane(qsq, 32);
        if ((SEL || STATS) && a.qn && g == 0 && tv) a.qn[rowbase + tok] = qsq;
        // this lane's output rows: tokens tw0 + 16 j + 4g + i
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qe[j][i] = __shfl(qsq, 4 * g + i, 64) + a.eps;
            rv[j][i] = tw0 + 16 * j + 4 * g + i < Tc;
        }
    }
    const FragBase<STORE, DHS> fb(r, g);
    // this lane's group of sixteen lanes (the lanes of one token row) in a
    // wavefront ballot, low and high words
    const uint32_t gm_lo = (g == 0) ? 0x0000ffffu : (g == 1 ? 0xffff0000u : 0u);
    const uint32_t gm_hi = (g == 2) ? 0x0000ffffu : (g == 3 ? 0xffff0000u : 0u);
    uint32_t ncand[TG][4];  // candidates appended so far to each of the lane's token lists

    float zinv[TG][4], zrow[TG][4], mrow[TG][4];  // 1/Z_t of the selection pass (0 past the chunk);
    uint32_t tau[TG][4];                          // Z_t from the workspace; dot scoring's row maximum M_t
#pragma unroll
    for (int j = 0; j < TG; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            zinv[j][i] = 0.f;
            zrow[j][i] = 1.f;
            mrow[j][i] = 0.f;
            tau[j][i] = 0u;
            ncand[j][i] = 0u;
        }
    if constexpr (ROW) {
        // log pbar_i from the per-tile usage partials, tiles added in order;
        // the first tile's workgroup also leaves it for the key step
        const float* pp = a.part + static_cast<size_t>(bhh) * a.pbar_ntiles * n;
        for (int i = threadIdx.x; i < n; i += 64 * NW) {
            const float l = log_pbar(pp, a.pbar_ntiles, n, i, Tc);
            lps[i] = l;
            if (tile == 0) a.lp[static_cast<size_t>(bhh) * n + i] = l;
        }
#pragma unroll
        for (int j = 0; j < TG; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (rv[j][i]) {
                    zrow[j][i] = a.Z[rowbase + tw0 + 16 * j + 4 * g + i];
                    if constexpr (DOT) mrow[j][i] = a.M[rowbase + tw0 + 16 * j + 4 * g + i];
                }
    }

#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        float zacc[TG][4], macc[TG][4];
        float zmax[TG][4];  // dot scoring's Z: a running maximum and the sum of exp(s - max) per lane
        uint32_t keep[TG][4][MK];
#pragma unroll
        for (int j = 0; j < TG; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                zacc[j][i] = 0.f;
                macc[j][i] = 0.f;
                zmax[j][i] = -INFINITY;
#pragma unroll
                for (int m = 0; m < MK; ++m) keep[j][i][m] = 0xffffffffu;
            }

        __syncthreads();  // the previous pass is done with kbuf
        dma_rows<CPR, KB, NW, false>(kbuf, Kg, CPR * 16, n, wave, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        for (int blk = 0; blk < nblk; ++blk) {
            const int cur = blk & 1;
            if (blk + 1 < nblk)
                dma_rows<CPR, KB, NW, false>(kbuf + (cur ^ 1) * BLK_BYTES, Kg + static_cast<size_t>(blk + 1) * KB * CPR * 16,
                                             CPR * 16, n - (blk + 1) * KB, wave, lane);
            const unsigned char* kb = kbuf + cur * BLK_BYTES;
            float colv[TG][KB / 16];
#pragma unroll
            for (int ct = 0; ct < KB / 16; ++ct) {
#pragma unroll
                for (int j = 0; j < TG; ++j) colv[j][ct] = 0.f;
                if (blk * KB + ct * 16 >= n) continue;  // partial last block (n % 16 == 0)
                const int key = blk * KB + ct * 16 + r;
                const float knv = DOT ? 0.f : kns[key];
                f32x4_t acc[TG];
#pragma unroll
                for (int j = 0; j < TG; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[j][i] = knv;
                // k-blocks in pairs, the next pair's LDS reads in flight under
                // this pair's MFMAs; each fragment feeds every group
                constexpr int NP = (DHS + 1) / 2;
                Frag<STORE> Bf[2][2];
                lds_frag<STORE, DHS>(Bf[0][0], kb, fb, ct, 0);
                if (DHS > 1) lds_frag<STORE, DHS>(Bf[0][1], kb, fb, ct, 1);
#pragma unroll
                for (int sp = 0; sp < NP; ++sp) {
                    if (sp + 1 < NP) {
                        lds_frag<STORE, DHS>(Bf[(sp + 1) & 1][0], kb, fb, ct, 2 * sp + 2);
                        lds_frag<STORE, DHS>(Bf[(sp + 1) & 1][1], kb, fb, ct, 2 * sp + 3);
                    }
#pragma unroll
                    for (int j = 0; j < TG; ++j) mma(A[j][2 * sp], Bf[sp & 1][0], acc[j]);
                    if (2 * sp + 1 < DHS)
#pragma unroll
                        for (int j = 0; j < TG; ++j) mma(A[j][2 * sp + 1], Bf[sp & 1][1], acc[j]);
                }
                if constexpr (STORE == kBF16) {
                    // keep two fragment reads in flight ahead of the MFMAs
                    // (left alone, the scheduler waits for each read just
                    // before its MFMA): the key norm and fragments 0 and 1
                    // first, then one read after each MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, DOT ? 2 : 3, 0);
#pragma unroll
                    for (int s = 0; s < DHS; ++s) {
                        __builtin_amdgcn_sched_group_barrier(0x008, TG, 0);
                        if (s + 2 < DHS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                }
                float lpk = 0.f;
                if constexpr (ROW) lpk = lps[key];
#pragma unroll
                for (int j = 0; j < TG; ++j) {
                    float cs = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // e = max(eps + d, eps): the large ||q||^2 enters with one
                        // rounding at the end; a signed-integer max of the bit
                        // patterns orders these floats exactly (eps > 0)
                        // dot scoring: smaller ord(-s) is better, p ~ exp(s - M)
                        const float x = acc[j][i];
                        const uint32_t eb = DOT ? ord_f32(-x)
                                                : static_cast<uint32_t>(max(__float_as_int(qe[j][i] + x), eps_bits));
                        const float e = __uint_as_float(eb);
                        if (pass == 0) {
                            if constexpr (STATS) {
                                if constexpr (DOT) {
                                    const float mx = fmaxf(zmax[j][i], x);
                                    zacc[j][i] = zacc[j][i] * __expf(zmax[j][i] - mx) + __expf(x - mx);
                                    zmax[j][i] = mx;
                                } else {
                                    zacc[j][i] += fast_rcp(e);
                                }
                            }
                            if constexpr (ROW)
                                macc[j][i] = fmaf(DOT ? __expf(x - mrow[j][i]) : fast_rcp(e), lpk, macc[j][i]);
                            if constexpr (SEL) {
                                // keep the MK smallest of this lane, ascending: with the
                                // list sorted, entry m becomes the median of (entry m-1,
                                // entry m, x) -- one v_med3_u32 each -- and entry 0 the
                                // smaller of itself and x (the same values as inserting
                                // x by compare-and-swap down the list)
#pragma unroll
                                for (int m = MK - 1; m >= 1; --m)
                                    keep[j][i][m] = med3_u32(keep[j][i][m - 1], keep[j][i][m], eb);
                                keep[j][i][0] = min(keep[j][i][0], eb);
                            }
                        } else {
                            if constexpr (STATS) cs = fmaf(DOT ? __expf(x - mrow[j][i]) : fast_rcp(e), zinv[j][i], cs);
                            if constexpr (SEL) {
                                // append (e, sub-key) to the token's list when e <= tau:
                                // positions from a ballot of the sixteen lanes of the
                                // token row, in lane (sub-key) order
                                const bool hit = eb <= tau[j][i];
                                const uint64_t m = ballot(hit);
                                if (m != 0u) {
                                    const uint32_t lo = static_cast<uint32_t>(m) & gm_lo;
                                    const uint32_t hi = static_cast<uint32_t>(m >> 32) & gm_hi;
                                    const uint32_t pos =
                                        ncand[j][i] + __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
                                    if (hit && pos < static_cast<uint32_t>(a.cap))
                                        a.cand[(rowbase + tw0 + 16 * j + 4 * g + i) * a.cap + pos] =
                                            (static_cast<uint64_t>(eb) << 32) | static_cast<uint32_t>(key);
                                    ncand[j][i] += __popc(lo) + __popc(hi);
                                }
                            }
                        }
                    }
                    colv[j][ct] = cs;
                }
            }
            if (STATS && pass == 1) {
                // sum over each group's 16 tokens: across the four lane groups
#pragma unroll
                for (int j = 0; j < TG; ++j)
#pragma unroll
                    for (int ct = 0; ct < KB / 16; ++ct) {
                        float x = colv[j][ct];
                        x += xor_lane(x, 16);
                        x += xor_lane(x, 32);
                        if (g == 0) colbuf[(cur * NG + wave * TG + j) * KB + ct * 16 + r] = x;
                    }
            }
            __builtin_amdgcn_s_waitcnt(0);  // this wave's part of the next block has landed
            __syncthreads();
            if (STATS && pass == 1 && threadIdx.x < KB && blk * KB + static_cast<int>(threadIdx.x) < n) {
                // this tile's partial of pbar for the block's sub-keys, groups in token order
                const float* cb = colbuf + cur * NG * KB + threadIdx.x;
                float s = cb[0];
#pragma unroll
                for (int w = 1; w < NG; ++w) s += cb[w * KB];
                a.part[(static_cast<size_t>(bhh) * ntiles + tile) * n + blk * KB + threadIdx.x] = s;
            }
        }

        if (pass == 0) {
#pragma unroll
            for (int j = 0; j < TG; ++j) {
                const size_t row0 = rowbase + tw0 + 16 * j + 4 * g;
                if constexpr (STATS) {
                    // Z_t over the sixteen lanes that share token 4g+i
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float x = zacc[j][i];
                        if constexpr (DOT) {
                            // merge (max, sum) pairs: sum' = sum e^(max - M) + sum2 e^(max2 - M)
                            float mx = zmax[j][i];
#pragma unroll
                            for (int o = 1; o <= 8; o <<= 1) {
                                const float m2 = xor_lane(mx, o), x2 = xor_lane(x, o);
                                const float M = fmaxf(mx, m2);
                                x = x * __expf(mx - M) + x2 * __expf(m2 - M);
                                mx = M;
                            }
                            mrow[j][i] = mx;
                            if (r == 0 && rv[j][i]) a.M[row0 + i] = mx;
                        } else {
                            x += xor_lane(x, 1);
                            x += xor_lane(x, 2);
                            x += xor_lane(x, 4);
                            x += xor_lane(x, 8);
                        }
                        zinv[j][i] = rv[j][i] ? fast_rcp(x) : 0.f;
                        if (r == 0 && rv[j][i]) a.Z[row0 + i] = x;
                    }
                }
                if constexpr (ROW) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float x = macc[j][i];
                        x += xor_lane(x, 1);
                        x += xor_lane(x, 2);
                        x += xor_lane(x, 4);
                        x += xor_lane(x, 8);
                        if (r == 0 && rv[j][i]) a.m[row0 + i] = x / zrow[j][i];
                    }
                }
                if constexpr (SEL) {
                    // tau = k'-th smallest of the 16*MK values kept by the token's lanes
                    constexpr int RS = (MK <= 1) ? 1 : (MK <= 2 ? 2 : 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t v[RS];
#pragma unroll
                        for (int m = 0; m < RS; ++m) v[m] = (m < MK) ? keep[j][i][m] : 0xffffffffu;
                        bitonic_sort<RS, 16>(v);
                        const int kth = a.kh - 1;
                        uint32_t t = 0u;
#pragma unroll
                        for (int m = 0; m < RS; ++m)
                            if (m == kth / 16) t = v[m];
                        t = static_cast<uint32_t>(__shfl(static_cast<int>(t), 16 * g + (kth % 16), 64));
                        tau[j][i] = rv[j][i] ? t : 0u;  // rows past the chunk collect nothing
                    }
                }
            }
        }
    }
    if constexpr (SEL) {
#pragma unroll
        for (int j = 0; j < TG; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (r == 0 && rv[j][i]) a.cnt[rowbase + tw0 + 16 * j + 4 * g + i] = static_cast<int32_t>(ncand[j][i]);
    }
}

// ---------------------------------------------------------------------------
// k_rows
// ---------------------------------------------------------------------------

// Scoring by whole rows, for chunks whose token tiles cannot fill the chip
// (decode; a single long sequence): every e_ti is written out so the
// selection takes an exact top-k' of whole rows and the addressing
// statistics are reductions over the stored rows.  One wavefront per
// (sequence, head, half, 16 sub-keys, 16 tokens): the sub-key rows are the
// MFMA's B operand, loaded straight from memory (wavefronts of the same
// sub-keys are adjacent, so the rereads hit L2).  The arithmetic
// (accumulators seeded with ||K_i||^2, -2q, k-blocks in order, ||q||^2 + eps
// added last) is that of k_score, so the e values are the same bits.
// Dot scoring writes ord(-s).  With a.qn the first sub-key block's
// wavefronts also write ||q_half||^2 of their tokens.
template <int STORE, int DHS, bool DOT>
__global__ __launch_bounds__(256) void k_rows(ScoreArgs a) {
    constexpr int ES = Store<STORE>::kBytes;
    const int n = a.n, H = a.H, Tc = a.Tc;
    const int kblk = n / 16, ttiles = (Tc + 15) / 16;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (gw >= static_cast<int64_t>(a.B) * H * 2 * kblk * ttiles) return;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int tt = static_cast<int>(gw % ttiles);
    const int64_t rest = gw / ttiles;
    const int kb = static_cast<int>(rest % kblk), bhh = static_cast<int>(rest / kblk);
    const int key = kb * 16 + r, t0 = tt * 16;
    const int half = bhh & 1, bh = bhh >> 1;
    const int h = bh % H, b = bh / H;
    Frag<STORE> Bf[DHS];
    load_row_frags<STORE, DHS>(Bf, static_cast<const unsigned char*>(half ? a.K2 : a.K1) +
                                       (static_cast<size_t>(bh) * n + key) * (32 * DHS) * ES, g);
    const float knv = DOT ? 0.f : a.knorm[static_cast<size_t>(bhh) * n + key];
    if constexpr (!DOT) {
        // -2 K rather than -2 q: the same exact products as the sweep's,
        // without a scaled copy of the query fragments beside the ones ||q||^2 reads
#pragma unroll
        for (int s = 0; s < DHS; ++s) frag_scale_m2(Bf[s]);
    }

    Frag<STORE> A[DHS];
    const int tok = t0 + r;
    const bool tv = tok < Tc;
    load_row_frags<STORE, DHS>(A, static_cast<const unsigned char*>(a.q) +
        (static_cast<size_t>(b) * a.q_bstride + static_cast<size_t>(tv ? tok : 0) * H * (64 * DHS) +
         h * (64 * DHS) + half * (32 * DHS)) * ES, g);
    float qsq = 0.f;
#pragma unroll
    for (int s = 0; s < DHS; ++s) {
        if (!tv) frag_zero<STORE>(A[s]);
        qsq += frag_sumsq<STORE>(A[s]);
    }
    qsq += xor_lane(qsq, 16);
    qsq += xor_lane(qsq, 32);
    const size_t rowbase = static_cast<size_t>(bhh) * Tc;
    if (a.qn && kb == 0 && g == 0 && tv) a.qn[rowbase + tok] = qsq;
    f32x4_t acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = knv;
#pragma unroll
    for (int s = 0; s < DHS; ++s) mma(A[s], Bf[s], acc);
    const int eps_bits = __float_as_int(a.eps);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + 4 * g + i;
        const float qe = __shfl(qsq, 4 * g + i, 64) + a.eps;
        const uint32_t eb = DOT ? ord_f32(-acc[i]) : static_cast<uint32_t>(max(__float_as_int(qe + acc[i]), eps_bits));
        if (t < Tc) a.erow[(rowbase + t) * n + key] = eb;
    }
}

// p_ti (without 1/Z_t) from a stored row entry: 1/e for IDW, exp(s - M_t) for dot.
template <bool DOT>
__device__ __forceinline__ float row_weight(uint32_t u, float M) {
    if constexpr (DOT) return __expf(-unord_f32(u) - M);
    else return fast_rcp(__uint_as_float(u));
}

// Row statistics of stored rows: Z_t = sum_i 1/e_ti (IDW), or M_t = max_i s_ti
// and Z_t = sum_i exp(s_ti - M_t) (dot).  One wavefront per row; each lane
// sums its sub-keys j*64 + lane in order, then an xor butterfly.
template <bool DOT>
__global__ __launch_bounds__(256) void k_row_z(ScoreArgs a) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // bhh*Tc + t
    if (row >= static_cast<int64_t>(a.B) * a.H * 2 * a.Tc) return;
    const int lane = threadIdx.x & 63, n = a.n;
    const uint32_t* e = a.erow + static_cast<size_t>(row) * n;
    uint32_t ev[kNplMax];
#pragma unroll
    for (int j = 0; j < kNplMax; ++j) ev[j] = (j * 64 + lane < n) ? e[j * 64 + lane] : 0u;
    float M = 0.f;
    if constexpr (DOT) {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kNplMax; ++j)
            if (j * 64 + lane < n) mx = fmaxf(mx, -unord_f32(ev[j]));
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, xor_lane(mx, o));
        M = mx;
    }
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < kNplMax; ++j)
        if (j * 64 + lane < n) z += row_weight<DOT>(ev[j], M);
    z = wave_sum(z);
    if (lane == 0) {
        a.Z[row] = z;
        if constexpr (DOT) a.M[row] = M;
    }
}

// Per-tile partial sums over tokens of p_ti for every sub-key (the pieces of
// the chunk's usage pbar), tiles of kScoreTokMin tokens.  One workgroup per
// (sequence, head, half, tile, 64 sub-keys): lane = sub-key, wavefront w sums
// tokens [16w, 16w + 16) of the tile in order, and the four wavefront sums
// are added in order.
template <bool DOT>
__global__ __launch_bounds__(256) void k_row_colsum(ScoreArgs a) {
    __shared__ float wsum[4][64];
    const int ntiles = (a.Tc + kScoreTokMin - 1) / kScoreTokMin;
    const int kblk = (a.n + 63) / 64;
    const int kb = blockIdx.x % kblk;
    const int tile = (blockIdx.x / kblk) % ntiles;
    const int bhh = blockIdx.x / (kblk * ntiles);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = a.n, i = kb * 64 + lane;
    const int t0 = tile * kScoreTokMin + wave * 16, t1 = min(a.Tc, t0 + 16);
    const size_t rowbase = static_cast<size_t>(bhh) * a.Tc;
    float s = 0.f;
    if (i < n) {
        // the wavefront's 16 tokens: every load in flight first, then the sum in token order
        uint32_t ev[16];
        float zv[16], mv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const size_t row = rowbase + min(t0 + u, a.Tc - 1);  // in the chunk; only t < t1 is summed
            ev[u] = a.erow[row * n + i];
            zv[u] = a.Z[row];
            mv[u] = DOT ? a.M[row] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (t0 + u < t1) s = fmaf(row_weight<DOT>(ev[u], mv[u]), fast_rcp(zv[u]), s);
    }
    wsum[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && i < n)
        a.part[(static_cast<size_t>(bhh) * ntiles + tile) * n + i] =
            ((wsum[0][lane] + wsum[1][lane]) + wsum[2][lane]) + wsum[3][lane];
}

// Row statistic m_t = sum_i p_ti ln pbar_i from stored rows.  One workgroup
// per kRowMRows rows of one (sequence, head, half): it first forms ln pbar
// from the usage partials in LDS (the first group also leaves it for the key
// step), then one wavefront per row.  Workgroups past a.stat_blocks write
// the chunk's transposed queries instead.
constexpr int kRowMRows = 16;
template <int STORE, bool DOT>
__global__ __launch_bounds__(64 * kRowMRows) void k_row_m(ScoreArgs a) {
    constexpr int LDS = kNplMax * 64 * 4 > qt_tile_bytes<STORE>() ? kNplMax * 64 * 4 : qt_tile_bytes<STORE>();
    __shared__ __align__(16) unsigned char lds[LDS];
    if (static_cast<int>(blockIdx.x) >= a.stat_blocks) {
        qt_tile_linear<STORE, kRowMRows>(a.qt, static_cast<int64_t>(blockIdx.x) - a.stat_blocks, lds);
        return;
    }
    float* lps = reinterpret_cast<float*>(lds);
    const int groups = (a.Tc + kRowMRows - 1) / kRowMRows;
    const int bhh = static_cast<int>(blockIdx.x / groups), grp = static_cast<int>(blockIdx.x % groups);
    const int lane = threadIdx.x & 63, n = a.n;
    {
        const float* pp = a.part + static_cast<size_t>(bhh) * a.pbar_ntiles * n;
        for (int i = threadIdx.x; i < n; i += 64 * kRowMRows) {
            const float l = log_pbar(pp, a.pbar_ntiles, n, i, a.Tc);
            lps[i] = l;
            if (grp == 0) a.lp[static_cast<size_t>(bhh) * n + i] = l;
        }
    }
    __syncthreads();
    const int t = grp * kRowMRows + (threadIdx.x >> 6);
    if (t >= a.Tc) return;
    const int64_t row = static_cast<int64_t>(bhh) * a.Tc + t;
    const uint32_t* e = a.erow + static_cast<size_t>(row) * n;
    const float* lp = lps;
    const float M = DOT ? a.M[row] : 0.f;
    // every load in flight first, then the sum over sub-keys lane, lane+64, ... in order
    uint32_t ev[kNplMax];
    float lv[kNplMax];
#pragma unroll
    for (int j = 0; j < kNplMax; ++j) {
        const bool in = j * 64 + lane < n;
        ev[j] = in ? e[j * 64 + lane] : 0u;
        lv[j] = in ? lp[j * 64 + lane] : 0.f;
    }
    float x = 0.f;
#pragma unroll
    for (int j = 0; j < kNplMax; ++j)
        if (j * 64 + lane < n) x = fmaf(row_weight<DOT>(ev[j], M), lv[j], x);
    x = wave_sum(x);
    if (lane == 0) a.m[row] = x / a.Z[row];
}

// ---------------------------------------------------------------------------
// k_select
// ---------------------------------------------------------------------------

// Exact top-kh smallest of a row (bit patterns of non-negative floats, +inf
// padding) by radix select on 8-bit digits, ties to the lower index.  Writes
// the winners unsorted as (value << 32 | index) keys to out[0..kh).
__device__ void radix_select(const uint32_t (&u)[kNplMax], int npl, int kh, uint32_t* hist, uint64_t* out) {
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
        const uint32_t cs[4] = {hist[4 * lane], hist[4 * lane + 1], hist[4 * lane + 2], hist[4 * lane + 3]};
        const uint32_t s = cs[0] + cs[1] + cs[2] + cs[3];
        uint32_t cb = wave_incl_scan_u32(s) - s;
        int found = -1;
        uint32_t fcb = 0u, fcnt = 0u;
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
            const bool pick = lt || (eq && er < need);
            const uint64_t sb = ballot(pick);
            const uint32_t pos = sel_base + __popcll(sb & lt_mask);
            if (pick) out[pos] = (static_cast<uint64_t>(x) << 32) | static_cast<uint32_t>(j * 64 + lane);
            eq_base += __popcll(eb);
            sel_base += __popcll(sb);
        }
    }
    wave_sync();
}

// Sorted top-kh (value, sub-key) of one (token, head, half) into out_e/out_i.
template <int STORE>
__device__ void half_topk(const SelectArgs& a, int b, int t, int h, int half, uint32_t* hist, uint64_t* buf,
                          float* out_e, int* out_i) {
    const int lane = lane_id();
    const int bhh = (b * a.H + h) * 2 + half;
    const size_t row = static_cast<size_t>(bhh) * a.Tc + t;
    const int count = a.cnt[row];
    uint64_t key[4];
    int R;
    if (count <= a.cap) {
        const uint64_t* c = a.cand + row * a.cap;
#pragma unroll
        for (int m = 0; m < 4; ++m) key[m] = (m * 64 + lane < count) ? c[m * 64 + lane] : ~0ull;
        R = count <= 64 ? 1 : (count <= 128 ? 2 : 4);
    } else {
        // exact distances of this row, then radix select
        const int dh = a.dh, n = a.n;
        const unsigned char* q = static_cast<const unsigned char*>(a.q) +
            (static_cast<size_t>(b) * a.q_bstride + (static_cast<size_t>(t) * a.H + h) * 2 * dh + half * dh) *
                Store<STORE>::kBytes;
        const void* K = half ? a.K2 : a.K1;
        const size_t kb = static_cast<size_t>(b * a.H + h) * n * dh;
        const int npl = (n + 63) >> 6;
        uint32_t u[kNplMax];
#pragma unroll
        for (int j = 0; j < kNplMax; ++j) {
            const int i = j * 64 + lane;
            u[j] = 0xffffffffu;
            if (j < npl && i < n) {
                float d = 0.f;
                for (int x = 0; x < dh; ++x) {
                    const float qx = ld_elem<STORE>(q, x), kx = ld_elem<STORE>(K, kb + static_cast<size_t>(i) * dh + x);
                    if (a.dot) {
                        d = fmaf(qx, kx, d);
                    } else {
                        const float diff = qx - kx;
                        d = fmaf(diff, diff, d);
                    }
                }
                u[j] = a.dot ? ord_f32(-d) : __float_as_uint(a.eps + d);
            }
        }
        radix_select(u, npl, a.kh, hist, buf);
#pragma unroll
        for (int m = 0; m < 4; ++m) key[m] = (m == 0 && lane < a.kh) ? buf[lane] : ~0ull;
        R = 1;
    }
    if (R == 1) {
        uint64_t k1[1] = {key[0]};
        bitonic_sort<1, 64>(k1);
        key[0] = k1[0];
    } else if (R == 2) {
        uint64_t k2[2] = {key[0], key[1]};
        bitonic_sort<2, 64>(k2);
        key[0] = k2[0];
    } else {
        bitonic_sort<4, 64>(key);
    }
    if (lane < a.kh) {
        const uint32_t kbits = static_cast<uint32_t>(key[0] >> 32);
        out_e[lane] = a.dot ? unord_f32(kbits) : __uint_as_float(kbits);
        out_i[lane] = static_cast<int>(key[0] & 0xffffffffu);
    }
    wave_sync();
}

// Sorted top-kh (value, sub-key) of one (token, head, half) from its whole
// row of e bit patterns (rows mode), ties to the lower index.  Each lane
// keeps its two smallest values; the kh-th smallest of those 128 is a bound
// tau with at least kh values of the row <= tau, so every value <= tau is a
// candidate (about kh of them) and one sort of the candidates finishes.
// More than 64 candidates (many equal values) fall back to a radix select.
// The loops run over all kNplMax entries of a lane without a branch (past
// the row's end a lane holds the padding ~0, which is never a candidate):
// a branch per entry made the wavefront wait for each candidate's LDS store
// at the join (measured in decode: the candidate pass 1.1 us of the 14.5).
__device__ void half_topk_row(const SelectArgs& a, size_t row, uint32_t* hist, uint64_t* buf, float* out_e,
                              int* out_i) {
    const int lane = lane_id();
    const int n = a.n, npl = (n + 63) >> 6;
    const uint32_t* e = a.erow + row * n;
    uint32_t u[kNplMax];
    uint32_t m0 = 0xffffffffu, m1 = 0xffffffffu;
#pragma unroll
    for (int j = 0; j < kNplMax; ++j) {
        const int i = j * 64 + lane;
        const uint32_t x = e[min(i, n - 1)];  // in bounds for every lane: no branch around the load
        u[j] = i < n ? x : 0xffffffffu;
        const uint32_t lo = min(m0, u[j]), hi = max(m0, u[j]);
        m0 = lo;
        m1 = min(m1, hi);
    }
    if (a.Z) {
        // the row statistics from the loaded row, in k_row_z's order
        float M = 0.f;
        if (a.dot) {
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < kNplMax; ++j) {
                const float sv = -unord_f32(u[j]);
                mx = j * 64 + lane < n ? fmaxf(mx, sv) : mx;
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, xor_lane(mx, o));
            M = mx;
        }
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < kNplMax; ++j) {
            const float wv = a.dot ? row_weight<true>(u[j], M) : row_weight<false>(u[j], 0.f);
            z = j * 64 + lane < n ? z + wv : z;
        }
        z = wave_sum(z);
        if (lane == 0) {
            a.Z[row] = z;
            if (a.dot) a.M[row] = M;
        }
    }
    uint32_t kept[2] = {m0, m1};
    bitonic_sort<2, 64>(kept);
    const uint32_t tau = static_cast<uint32_t>(__shfl(static_cast<int>(kept[0]), a.kh - 1, 64));  // kh <= 64
    const uint64_t lt = lanemask_lt();
    uint32_t total = 0u;
#pragma unroll
    for (int j = 0; j < kNplMax; ++j) {
        const bool c = u[j] <= tau && j * 64 + lane < n;
        const uint64_t bm = ballot(c);
        const uint32_t pos = total + static_cast<uint32_t>(__popcll(bm & lt));
        if (c && pos < 64u) buf[pos] = (static_cast<uint64_t>(u[j]) << 32) | static_cast<uint32_t>(j * 64 + lane);
        total += static_cast<uint32_t>(__popcll(bm));
    }
    wave_sync();
    uint64_t key[1];
    if (total <= 64u) {
        key[0] = (static_cast<uint32_t>(lane) < total) ? buf[lane] : ~0ull;
    } else {
        wave_sync();
        radix_select(u, npl, a.kh, hist, buf);
        key[0] = (lane < a.kh) ? buf[lane] : ~0ull;
    }
    bitonic_sort<1, 64>(key);
    if (lane < a.kh) {
        const uint32_t kbits = static_cast<uint32_t>(key[0] >> 32);
        out_e[lane] = a.dot ? unord_f32(kbits) : __uint_as_float(kbits);
        out_i[lane] = static_cast<int>(key[0] & 0xffffffffu);
    }
    wave_sync();
}

// The product candidates' rank pairs of this lane: entry r is candidate
// r*64 + lane (a*64 + b of its two per-half ranks; entries past ncand are
// not used).  Loaded apart from the product top-k, without a condition, so
// that a caller can request it early and wait for it only where it is used.
__device__ __forceinline__ void load_ab(const SelectArgs& a, uint32_t (&ab)[kMaxCand / 64]) {
    const int lane = lane_id();
#pragma unroll
    for (int r = 0; r < kMaxCand / 64; ++r) ab[r] = a.cand_ab.ab[r * 64 + lane];
}

template <int R>
__device__ void product_topk(const SelectArgs& a, const float* e1, const int* i1, const float* e2, const int* i2,
                             int32_t* idx_out, float* w_out, int32_t* usage, const uint32_t (&abr)[kMaxCand / 64]) {
    const int lane = lane_id();
    uint64_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int c = r * 64 + lane;
        if (c < a.ncand) {
            const uint32_t ab = abr[r];
            const int ia = static_cast<int>(ab >> 6), ib = static_cast<int>(ab & 63u);
            // IDW: P = (eps + d1)(eps + d2); dot: v = -(s1 + s2); smaller is better
            const float P = a.dot ? e1[ia] + e2[ib] : e1[ia] * e2[ib];
            const uint32_t slot = static_cast<uint32_t>(i1[ia] * a.n + i2[ib]);
            key[r] = (static_cast<uint64_t>(a.dot ? ord_f32(P) : __float_as_uint(P)) << 32) | slot;
        } else {
            key[r] = ~0ull;
        }
    }
    bitonic_sort<R, 64>(key);
    const uint32_t pbits = static_cast<uint32_t>(key[0] >> 32);
    const float P = a.dot ? unord_f32(pbits) : __uint_as_float(pbits);
    const float P0 = __shfl(P, 0, 64);
    // w = softmax of the k pair scores: (1/P)/sum(1/P) for IDW, exp(-v)/sum for dot
    const float ratio = (lane < a.k) ? (a.dot ? __expf(P0 - P) : (P0 / P)) : 0.f;
    const float sum = wave_sum(ratio);
    if (lane < a.k) {
        const int32_t slot = static_cast<int32_t>(key[0] & 0xffffffffu);
        idx_out[lane] = slot;
        w_out[lane] = ratio / sum;
        // row contribution of this read (integer atomic: exact in any order)
        if (usage && slot >= 0 && slot < a.n * a.n) atomicAdd(usage + slot, 1);
    }
}

// The product top-k of one (token, head) with the register width its
// candidate count needs.
__device__ __forceinline__ void product_topk_n(const SelectArgs& a, const float* e1, const int* i1, const float* e2,
                                               const int* i2, int32_t* idx_out, float* w_out, int32_t* usage,
                                               const uint32_t (&ab)[kMaxCand / 64]) {
    if (a.ncand <= 64) product_topk<1>(a, e1, i1, e2, i2, idx_out, w_out, usage, ab);
    else if (a.ncand <= 128) product_topk<2>(a, e1, i1, e2, i2, idx_out, w_out, usage, ab);
    else product_topk<4>(a, e1, i1, e2, i2, idx_out, w_out, usage, ab);
}

// Items (token, head) of a launch from which the rare-path items get a
// launch of their own (measured: 32768 items, the million batch, gain 1.2%;
// 16384, collision, and 8192, mid, lose about as much to the extra launch).
constexpr int64_t kSelectSplitItems = 32768;

// Both candidate lists of an item fit one 64-wide register (the usual case).
__device__ __forceinline__ bool lists_fit(const SelectArgs& a, int c0, int c1) {
    return c0 <= 64 && c1 <= 64 && a.cap >= 64;
}

// The items whose candidate lists do not fit one register (a list over 64
// entries, or over its capacity): exact top-k' of each half by recompute and
// radix select, then the product top-k, as k_select would.  A separate
// kernel so that k_select, which nearly every item takes, does not carry this
// path's registers.  Each wavefront checks 64 consecutive items and takes
// the ones that did not fit, in order; it usually finds none.
template <int STORE>
__global__ __launch_bounds__(256) void k_select_ovf(SelectArgs a) {
    __shared__ uint64_t buf[4][64];
    __shared__ uint32_t hist[4][256];
    __shared__ float se[4][2][kMaxKHalf];
    __shared__ int si[4][2][kMaxKHalf];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t items = static_cast<int64_t>(a.B) * a.Tc * a.H;
    const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * 64;
    bool ovf = false;
    if (i0 + lane < items) {
        const int64_t item = i0 + lane;
        const int h = static_cast<int>(item % a.H);
        const int64_t bt = item / a.H;
        const int t = static_cast<int>(bt % a.Tc), b = static_cast<int>(bt / a.Tc);
        const size_t row0 = (static_cast<size_t>(b * a.H + h) * 2) * a.Tc + t;
        ovf = !lists_fit(a, a.cnt[row0], a.cnt[row0 + a.Tc]);
    }
    uint64_t todo = ballot(ovf);
    while (todo) {
        const int l = __ffsll(static_cast<unsigned long long>(todo)) - 1;
        todo &= todo - 1;
        const int64_t item = i0 + l;
        const int h = static_cast<int>(item % a.H);
        const int64_t bt = item / a.H;
        const int t = static_cast<int>(bt % a.Tc), b = static_cast<int>(bt / a.Tc);
        for (int half = 0; half < 2; ++half)
            half_topk<STORE>(a, b, t, h, half, hist[wave], buf[wave], se[wave][half], si[wave][half]);
        const size_t o = static_cast<size_t>(b) * a.iw_bstride + (static_cast<size_t>(t) * a.H + h) * a.k;
        int32_t* u = a.usage ? a.usage + static_cast<size_t>(b) * a.n * a.n : nullptr;
        uint32_t ab[kMaxCand / 64];
        load_ab(a, ab);
        product_topk_n(a, se[wave][0], si[wave][0], se[wave][1], si[wave][1], a.idx + o, a.w + o, u, ab);
        wave_sync();
    }
}

// INLINE: the items whose lists do not fit are taken here too; otherwise
// they are left to k_select_ovf (chosen per launch by the item count).
template <int STORE, bool INLINE>
__global__ __launch_bounds__(256) void k_select(SelectArgs a) {
    __shared__ uint64_t buf[INLINE ? 4 : 1][64];
    __shared__ uint32_t hist[INLINE ? 4 : 1][256];
    __shared__ float se[4][2][kMaxKHalf];
    __shared__ int si[4][2][kMaxKHalf];
    const int wave = threadIdx.x >> 6;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + wave;  // over B*Tc*H
    if (item >= static_cast<int64_t>(a.B) * a.Tc * a.H) return;
    const int h = static_cast<int>(item % a.H);
    const int64_t bt = item / a.H;
    const int t = static_cast<int>(bt % a.Tc), b = static_cast<int>(bt / a.Tc);
    const size_t row0 = (static_cast<size_t>(b * a.H + h) * 2) * a.Tc + t;  // half 0; half 1 is Tc further
    const int c0 = a.cnt[row0], c1 = a.cnt[row0 + a.Tc];
    uint32_t ab[kMaxCand / 64];
    load_ab(a, ab);  // requested with the list counts, used after the sort
    if (lists_fit(a, c0, c1)) {
        // the usual case: both lists fit one register; sort them together
        const int lane = threadIdx.x & 63;
        uint64_t key[2];
        key[0] = (lane < c0) ? a.cand[row0 * a.cap + lane] : ~0ull;
        key[1] = (lane < c1) ? a.cand[(row0 + a.Tc) * a.cap + lane] : ~0ull;
        bitonic_sort_lists<2>(key);
        if (lane < a.kh) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t kbits = static_cast<uint32_t>(key[half] >> 32);
                se[wave][half][lane] = a.dot ? unord_f32(kbits) : __uint_as_float(kbits);
                si[wave][half][lane] = static_cast<int>(key[half] & 0xffffffffu);
            }
        }
        wave_sync();
    } else {
        if constexpr (!INLINE) return;  // k_select_ovf takes this item
        for (int half = 0; half < 2; ++half)
            half_topk<STORE>(a, b, t, h, half, hist[INLINE ? wave : 0], buf[INLINE ? wave : 0], se[wave][half],
                             si[wave][half]);
    }
    const size_t o = static_cast<size_t>(b) * a.iw_bstride + (static_cast<size_t>(t) * a.H + h) * a.k;
    int32_t* u = a.usage ? a.usage + static_cast<size_t>(b) * a.n * a.n : nullptr;
    product_topk_n(a, se[wave][0], si[wave][0], se[wave][1], si[wave][1], a.idx + o, a.w + o, u, ab);
}

// Selection from whole rows (rows mode, a few tokens): two wavefronts per
// (token, head), one per half, then the first does the product top-k.
__global__ __launch_bounds__(256) void k_select_rows(SelectArgs a) {
    __shared__ uint64_t buf[4][64];
    __shared__ uint32_t hist[4][256];
    __shared__ float se[2][2][kMaxKHalf];
    __shared__ int si[2][2][kMaxKHalf];
    const int wave = threadIdx.x >> 6, slot = wave >> 1, half = wave & 1;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 2 + slot;  // over B*Tc*H
    const bool live = item < static_cast<int64_t>(a.B) * a.Tc * a.H;
    uint32_t ab[kMaxCand / 64];
    load_ab(a, ab);  // requested before the row, used by the product top-k
    int b = 0, t = 0, h = 0;
    if (live) {
        h = static_cast<int>(item % a.H);
        const int64_t bt = item / a.H;
        t = static_cast<int>(bt % a.Tc);
        b = static_cast<int>(bt / a.Tc);
        const size_t row = ((static_cast<size_t>(b * a.H + h) * 2) + half) * a.Tc + t;
        half_topk_row(a, row, hist[wave], buf[wave], se[slot][half], si[slot][half]);
    }
    __syncthreads();
    if (!live || half != 0) return;
    const size_t o = static_cast<size_t>(b) * a.iw_bstride + (static_cast<size_t>(t) * a.H + h) * a.k;
    int32_t* u = a.usage ? a.usage + static_cast<size_t>(b) * a.n * a.n : nullptr;
    product_topk_n(a, se[slot][0], si[slot][0], se[slot][1], si[slot][1], a.idx + o, a.w + o, u, ab);
}

// Decode: one token's selection and read in one workgroup.  Wavefront 2h+half
// takes the top-k' of row (h, half); wavefront h < H then the product top-k
// of head h, written to idx / w; then one wavefront per part of the H*k
// entries reads the value rows (gather_token_split).  The same device code in
// the same order as k_select_rows followed by k_gather_split, so the same bits,
// with one launch fewer on a path where a launch is a large part of a token.
// The selection's scratch and the read's parts are never live together.
// What does not depend on the selection is requested before it, by every
// wavefront and without a condition (clamped to valid addresses), so that
// nothing waits for it before its use: the product table, the epilogue's g
// and v row (used by wavefront 0) and kSgCopy 16-byte pieces per thread of
// the stream's copies into the pending chunk, stored after the row
// selection (pieces beyond those by a loop).  Measured per decode call of
// the 2^20-slot layer (16 tokens, 4 heads): the epilogue's dependent loads
// and copies had taken 2.4 us and the read's second round trip 1.3 us of
// the kernel's 14.5 us.  A stream launch only (ga.pq set).
constexpr int kSgScratch = (kSgWaves * 64 * 8 + kSgWaves * 256 * 4) > (kSgWaves * 512 * 4)
                               ? (kSgWaves * 64 * 8 + kSgWaves * 256 * 4) : (kSgWaves * 512 * 4);

template <int STORE, int EPL>
__global__ __launch_bounds__(64 * kSgWaves) void k_select_gather(SelectArgs a, GatherArgs ga) {
    __shared__ __align__(16) unsigned char scratch[kSgScratch];
    __shared__ float se[kSgWaves / 2][2][kMaxKHalf];
    __shared__ int si[kSgWaves / 2][2][kMaxKHalf];
    uint64_t (*buf)[64] = reinterpret_cast<uint64_t (*)[64]>(scratch);
    uint32_t (*hist)[256] = reinterpret_cast<uint32_t (*)[256]>(scratch + kSgWaves * 64 * 8);
    float (*part)[512] = reinterpret_cast<float (*)[512]>(scratch);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t tok = blockIdx.x;  // b*Tc + t
    const int t = static_cast<int>(tok % a.Tc), b = static_cast<int>(tok / a.Tc);
    uint32_t ab[kMaxCand / 64];
    load_ab(a, ab);
    const float gt = ga.g[static_cast<size_t>(b) * ga.g_bstride + t];
    RawRow<STORE, EPL> vraw;
    ld_raw_row<STORE, EPL>(ga.v, static_cast<size_t>(b) * ga.v_bstride + static_cast<size_t>(t) * ga.dv +
                                     static_cast<size_t>(lane) * EPL, vraw);
    const int npieces = pending_pieces<STORE>(ga, t);  // >= 1: q is never empty
    const int w0 = threadIdx.x, w1 = threadIdx.x + static_cast<int>(blockDim.x);
    const uint4 cp0 = *pending_src<STORE>(ga, b, t, min(w0, npieces - 1));
    const uint4 cp1 = *pending_src<STORE>(ga, b, t, min(w1, npieces - 1));
    if (wave < 2 * a.H) {
        const int h = wave >> 1, half = wave & 1;
        const size_t row = ((static_cast<size_t>(b * a.H + h) * 2) + half) * a.Tc + t;
        half_topk_row(a, row, hist[wave], buf[wave], se[h][half], si[h][half]);
    }
    if (w0 < npieces) *pending_dst<STORE>(ga, b, t, w0) = cp0;
    if (w1 < npieces) *pending_dst<STORE>(ga, b, t, w1) = cp1;
    pending_copy<STORE>(ga, b, t, w1 + static_cast<int>(blockDim.x), static_cast<int>(blockDim.x));
    if (threadIdx.x == 0) ga.pg[static_cast<size_t>(b) * ga.pg_bstride + t] = gt;
    __syncthreads();
    if (wave < a.H) {
        const int h = wave;
        const size_t o = static_cast<size_t>(b) * a.iw_bstride + (static_cast<size_t>(t) * a.H + h) * a.k;
        int32_t* u = a.usage ? a.usage + static_cast<size_t>(b) * a.n * a.n : nullptr;
        product_topk_n(a, se[h][0], si[h][0], se[h][1], si[h][1], a.idx + o, a.w + o, u, ab);
    }
    __syncthreads();  // the slot lists are visible to the workgroup; the scratch is free
    FinishIn<EPL> fin;
    fin.gt = gt;
    widen_raw_row<STORE, EPL>(vraw, fin.vt);
    gather_token_split<STORE, EPL>(ga, tok, part, &fin);
}

template <int STORE, int DHS, int MK, int MODE, int NW, int TG, bool DOT>
hipError_t score_w(const ScoreArgs& a, hipStream_t s) {
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int KB = kKB<STORE, NW>;
    constexpr int NG = NW * TG;
    constexpr size_t BLK_BYTES = static_cast<size_t>(KB) * DHS * 32 * ES;
    const size_t lds = 2 * BLK_BYTES + static_cast<size_t>(a.n) * 4 + ((MODE & kScoreStats) ? 2 * NG * KB * 4 : 0) +
                       ((MODE & kScoreRowStat) ? static_cast<size_t>(a.n) * 4 : 0);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_score<STORE, DHS, MK, MODE, NW, TG, DOT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int ntiles = (a.Tc + 16 * NG - 1) / (16 * NG);
    const unsigned grid = static_cast<unsigned>(a.B * a.H * 2 * ntiles);
    hipLaunchKernelGGL((k_score<STORE, DHS, MK, MODE, NW, TG, DOT>), dim3(grid), dim3(64 * NW), lds, s, a);
    return hipGetLastError();
}

template <int STORE, int DHS, int MK, int MODE>
hipError_t score_t(const ScoreArgs& a, hipStream_t s) {
    // dot-product scoring (an ablation) is built for 64-token tiles only
    if (a.dot) return score_w<STORE, DHS, MK, MODE, 4, 1, true>(a, s);
    switch (a.tile) {
        case 64: return score_w<STORE, DHS, MK, MODE, 4, 1, false>(a, s);
        case 128: return score_w<STORE, DHS, MK, MODE, 8, 1, false>(a, s);
        case 256: return score_w<STORE, DHS, MK, MODE, 16, 1, false>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int STORE, int DHS, int MK>
hipError_t score_mode(const ScoreArgs& a, hipStream_t s) {
    switch (a.mode) {
        case kScoreSelect: return score_t<STORE, DHS, MK, kScoreSelect>(a, s);
        case kScoreSelect | kScoreStats: return score_t<STORE, DHS, MK, kScoreSelect | kScoreStats>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int STORE, int DHS>
hipError_t score_mk(const ScoreArgs& a, hipStream_t s) {
    if (a.mode == kScoreRows) {
        const int64_t waves = static_cast<int64_t>(a.B) * a.H * 2 * (a.n / 16) * ((a.Tc + 15) / 16);
        if (a.dot)
            hipLaunchKernelGGL((k_rows<STORE, DHS, true>), dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_rows<STORE, DHS, false>), dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    // modes without selection do not keep per-lane minima
    if (a.mode == kScoreStats) return score_t<STORE, DHS, 1, kScoreStats>(a, s);
    if (a.mode == kScoreRowStat) return score_t<STORE, DHS, 1, kScoreRowStat>(a, s);
    switch (score_keep(a.kh)) {
        case 2: return score_mode<STORE, DHS, 2>(a, s);
        case 3: return score_mode<STORE, DHS, 3>(a, s);
        case 4: return score_mode<STORE, DHS, 4>(a, s);
    }
    return hipErrorInvalidValue;
}

template <int STORE>
hipError_t score_s(const ScoreArgs& a, hipStream_t s) {
    switch (a.dh / 32) {
        case 1: return score_mk<STORE, 1>(a, s);
        case 2: return score_mk<STORE, 2>(a, s);
        case 4: return score_mk<STORE, 4>(a, s);
        case 8: return score_mk<STORE, 8>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int score_keep(int kh) {
    const int mk = (kh + 15) / 16 + 1;
    return mk > 4 ? 4 : mk;
}

int score_cap(int kh) { return kh <= 32 ? 128 : 256; }

int score_tile(int B, int H, int Tc, bool dot) {
    if (dot) return kScoreTokMin;  // the dot-product variant is built for 64-token tiles
    const int ncu = device_cus();
    const int span = (Tc + 15) / 16 * 16;  // no wider than the chunk
    for (int tile = kScoreTokMax; tile > kScoreTokMin; tile >>= 1) {
        if (tile > span) continue;
        const long long wgs = static_cast<long long>(B) * H * 2 * ((Tc + tile - 1) / tile);
        if (wgs >= ncu) return tile;
    }
    return kScoreTokMin;
}

hipError_t launch_row_stats(const ScoreArgs& a, int what, int store, hipStream_t s) {
    const int64_t rows = static_cast<int64_t>(a.B) * a.H * 2 * a.Tc;
    const unsigned rgrid = static_cast<unsigned>((rows + 3) / 4);
    if (what == 0 || what == 2) {  // Z (and M) unless the selection left them, then the usage partials
        const int ntiles = (a.Tc + kScoreTokMin - 1) / kScoreTokMin;
        const unsigned cgrid = static_cast<unsigned>(a.B * a.H * 2 * ntiles * ((a.n + 63) / 64));
        if (a.dot) {
            if (what == 0) hipLaunchKernelGGL(k_row_z<true>, dim3(rgrid), dim3(256), 0, s, a);
            hipLaunchKernelGGL(k_row_colsum<true>, dim3(cgrid), dim3(256), 0, s, a);
        } else {
            if (what == 0) hipLaunchKernelGGL(k_row_z<false>, dim3(rgrid), dim3(256), 0, s, a);
            hipLaunchKernelGGL(k_row_colsum<false>, dim3(cgrid), dim3(256), 0, s, a);
        }
    } else {  // the row statistic m (and the transposed queries)
        ScoreArgs b = a;
        b.stat_blocks = a.B * a.H * 2 * ((a.Tc + kRowMRows - 1) / kRowMRows);
        const unsigned mgrid = static_cast<unsigned>(b.stat_blocks + (a.qt.qT ? qt_tiles(a.qt) : 0));
        const dim3 blk(64 * kRowMRows);
        if (store == kBF16) {
            if (a.dot) hipLaunchKernelGGL((k_row_m<kBF16, true>), dim3(mgrid), blk, 0, s, b);
            else hipLaunchKernelGGL((k_row_m<kBF16, false>), dim3(mgrid), blk, 0, s, b);
        } else {
            if (a.dot) hipLaunchKernelGGL((k_row_m<kF32, true>), dim3(mgrid), blk, 0, s, b);
            else hipLaunchKernelGGL((k_row_m<kF32, false>), dim3(mgrid), blk, 0, s, b);
        }
    }
    return hipGetLastError();
}

int device_cus() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int v = 0;
        cus[dev] = (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
                       ? v : 256;
    }
    return cus[dev];
}

hipError_t launch_score(const ScoreArgs& a, int store, hipStream_t s) {
    ScoreArgs b = a;
    b.tile = score_tile(a.B, a.H, a.Tc, a.dot != 0);
    return store == kBF16 ? score_s<kBF16>(b, s) : score_s<kF32>(b, s);
}

bool select_gather_fits(int H, int k) {
    return 2 * H <= kSgWaves && (H * k + kGatherPart - 1) / kGatherPart <= kSgWaves;
}

template <int STORE>
hipError_t select_gather_s(const SelectArgs& a, const GatherArgs& ga, hipStream_t s) {
    const int nparts = (a.H * a.k + kGatherPart - 1) / kGatherPart;
    const int nw = max(2 * a.H, nparts);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Tc)), block(64 * nw);
    switch (ga.dv / 64) {
        case 1: hipLaunchKernelGGL((k_select_gather<STORE, 1>), grid, block, 0, s, a, ga); break;
        case 2: hipLaunchKernelGGL((k_select_gather<STORE, 2>), grid, block, 0, s, a, ga); break;
        case 4: hipLaunchKernelGGL((k_select_gather<STORE, 4>), grid, block, 0, s, a, ga); break;
        case 8: hipLaunchKernelGGL((k_select_gather<STORE, 8>), grid, block, 0, s, a, ga); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_select_gather(const SelectArgs& a, const GatherArgs& ga, int store, hipStream_t s) {
    if (!a.erow || !ga.pq || !ga.o || ga.r || !select_gather_fits(a.H, a.k) || a.B != ga.B || a.Tc != ga.Tc)
        return hipErrorInvalidValue;
    return store == kBF16 ? select_gather_s<kBF16>(a, ga, s) : select_gather_s<kF32>(a, ga, s);
}

hipError_t launch_select(const SelectArgs& a, int store, hipStream_t s) {
    const int64_t items = static_cast<int64_t>(a.B) * a.Tc * a.H;
    if (a.erow) {
        hipLaunchKernelGGL(k_select_rows, dim3(static_cast<unsigned>((items + 1) / 2)), dim3(256), 0, s, a);
        return hipGetLastError();
    }
    const unsigned grid = static_cast<unsigned>((items + 3) / 4);
    const unsigned ogrid = static_cast<unsigned>((items + 255) / 256);  // 64 items per wavefront
    // Many items: the usual path alone (27 registers instead of over 100)
    // and the rare one in a launch of its own, which leaves the value path
    // more of the chip (million: 8.08 -> 7.98 ms per step).  Fewer items: the
    // extra launch costs about what it gives back (mid: 2.29 -> 2.31 ms).
    const bool split = items >= kSelectSplitItems;
    if (store == kBF16) {
        if (split) {
            hipLaunchKernelGGL((k_select<kBF16, false>), dim3(grid), dim3(256), 0, s, a);
            hipLaunchKernelGGL(k_select_ovf<kBF16>, dim3(ogrid), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((k_select<kBF16, true>), dim3(grid), dim3(256), 0, s, a);
        }
    } else {
        if (split) {
            hipLaunchKernelGGL((k_select<kF32, false>), dim3(grid), dim3(256), 0, s, a);
            hipLaunchKernelGGL(k_select_ovf<kF32>, dim3(ogrid), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL((k_select<kF32, true>), dim3(grid), dim3(256), 0, s, a);
        }
    }
    return hipGetLastError();
}

}  // namespace fwpkm
