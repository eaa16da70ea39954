// k_score.hip -- sub-key scoring of a chunk against both half codebooks.
//
// Scoring ("Fast-weight Product Key Memory": paperlayer.ai 2.2 and A.2,
// rainbus digest step 2): the query is split into halves and each half is
// compared with every sub-key of its codebook by squared Euclidean distance,
// computed as ||q||^2 + ||K_i||^2 - 2 q.K_i on the matrix cores; the score
// is s = -log(eps + d).  Statistics of the addressing step (digest step 5,
// paperlayer.ai 3.4) use p_ti = (1/e_ti) / Z_t, e = eps + d, Z_t = sum_i 1/e_ti.
//
// k_score streams the codebook through LDS like a GEMM: a workgroup owns 64
// tokens of one (sequence, head) -- 16 per wavefront, the MFMA rows -- and
// walks the sub-keys in blocks of kKB, double-buffered, so every sub-key row
// is read from L2 once per 64 tokens.  Nothing of the distance matrix is
// stored; each mode reduces it in registers:
//
//  kScoreSelect   pass 1: Z_t, and for each lane the MK smallest e of the
//                 sub-keys it sees; tau_t = k'-th smallest of those 16*MK
//                 values is an upper bound of the k'-th smallest e of the row
//                 (at least k' values are <= tau_t).  Pass 2 recomputes the
//                 tile and appends every (e, sub-key) with e <= tau_t to the
//                 token's candidate list in the workspace; k_select then
//                 sorts the few candidates.
//  kScoreStats    pass 2 also forms the per-64-token partial sums over tokens
//                 of p_ti, the pieces of the chunk's marginal usage pbar.
//  kScoreRowStat  one pass: Z_t and m_t = sum_i p_ti log pbar_i.
//
// k_select: one wavefront per (token, head): sorts each half's candidates
// by (e, sub-key) for the top-k' (ties to the lower sub-key index), then the
// top-k of the product candidates by P = e1*e2 (ties to the lower slot id
// i*n + j) and the weights (1/P)/sum(1/P) = softmax of s1 + s2.  A token
// whose candidate list overflowed recomputes its distances exactly and
// selects by radix select.
#include "mfma_frag.h"

namespace fwpkm {

namespace {

// sub-keys per LDS block: 32 bf16 or 16 fp32 rows (at most 16 KiB for d_h <= 256)
template <int STORE> constexpr int kKB = (STORE == kBF16) ? 32 : 16;
constexpr int kTok = 64;       // tokens per k_score workgroup
constexpr int kNplMax = 16;    // sub-keys per lane in a row: n <= 1024

__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(x), m, 64);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(x >> 32), m, 64);
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
                        const bool sw = up ? (a > b) : (a < b);
                        x[r] = sw ? b : a;
                        x[r2] = sw ? a : b;
                    }
                }
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    K y;
                    if constexpr (sizeof(K) == 8) y = shfl_xor_u64(x[r], stride);
                    else y = __shfl_xor(x[r], stride, 64);
                    const int p = r * W + ln;
                    const bool up = (p & size) == 0;
                    const bool lower = (ln & stride) == 0;
                    const K mn = x[r] < y ? x[r] : y;
                    const K mx = x[r] < y ? y : x[r];
                    x[r] = (lower == up) ? mn : mx;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// k_score
// ---------------------------------------------------------------------------
template <int STORE, int DHS, int MK>
__global__ __launch_bounds__(256) void k_score(ScoreArgs a) {
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int PADK = 16 / ES;  // LDS row padding (elements): 16 bytes
    constexpr int KB = kKB<STORE>;
    extern __shared__ __align__(16) unsigned char smem[];
    const int n = a.n, H = a.H, dh = a.dh;
    const int kstride = dh + PADK;
    unsigned char* kbuf = smem;                                                  // [2][KB][kstride]
    float* colbuf = reinterpret_cast<float*>(kbuf + 2 * KB * kstride * ES);     // [2][4][KB]
    float* lps = colbuf + 2 * 4 * KB;                                            // [n] (rowstat)

    const int ntiles = (a.Tc + kTok - 1) / kTok;
    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = static_cast<int>(lid % ntiles);
    const int bh = static_cast<int>(lid / ntiles);
    const int h = bh % H, b = bh / H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int tw0 = tile * kTok + wave * 16;       // first token of this wavefront
    const int dq = 2 * dh;
    const bool sel = (a.mode & kScoreSelect) != 0;
    const bool stats = (a.mode & kScoreStats) != 0;
    const bool rowstat = (a.mode & kScoreRowStat) != 0;
    const int npass = (sel || stats) ? 2 : 1;
    const int nblk = (n + KB - 1) / KB;
    // cooperative block load: each thread moves 16-byte pieces of a block
    const int row_pieces = dh * ES / 16;            // 16-byte pieces per sub-key row
    const int blk_pieces = KB * row_pieces;
    const int my_pieces = (blk_pieces + 255) / 256; // <= 4

    for (int half = 0; half < 2; ++half) {
        const int bhh = (b * H + h) * 2 + half;
        const unsigned char* Kg = static_cast<const unsigned char*>(half ? a.K2 : a.K1) +
                                  static_cast<size_t>(b * H + h) * n * dh * ES;
        const float* kn = a.knorm + static_cast<size_t>(bhh) * n;
        // query fragments: token tw0 + r of this half (zero past the chunk)
        Frag<STORE> A[DHS];
        const int tok = tw0 + r;
        const bool tv = tok < a.Tc;
        const unsigned char* qrow = static_cast<const unsigned char*>(a.q) +
            (static_cast<size_t>(b) * a.q_bstride + static_cast<size_t>(tv ? tok : 0) * H * dq + h * dq + half * dh) * ES;
        load_row_frags<STORE, DHS>(A, qrow, g);
        float qsq = 0.f;
#pragma unroll
        for (int s = 0; s < DHS; ++s) {
            if (!tv) frag_zero<STORE>(A[s]);
            qsq += frag_sumsq<STORE>(A[s]);
        }
        qsq += __shfl_xor(qsq, 16, 64);
        qsq += __shfl_xor(qsq, 32, 64);
        if (a.qn && (sel || stats) && g == 0 && tv) a.qn[static_cast<size_t>(bhh) * a.Tc + tok] = qsq;
        // this lane's output rows: tokens tw0 + 4g + i
        float qn_row[4];
        bool rv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qn_row[i] = __shfl(qsq, 4 * g + i, 64);
            rv[i] = tw0 + 4 * g + i < a.Tc;
        }
        if (rowstat) {
            __syncthreads();
            for (int i = threadIdx.x; i < n; i += 256) lps[i] = a.lp[static_cast<size_t>(bhh) * n + i];
        }

        float zinv[4] = {0.f, 0.f, 0.f, 0.f};
        uint32_t tau[4] = {0u, 0u, 0u, 0u};
        for (int pass = 0; pass < npass; ++pass) {
            const bool last = pass == npass - 1;
            float zacc[4] = {0.f, 0.f, 0.f, 0.f}, macc[4] = {0.f, 0.f, 0.f, 0.f};
            uint32_t keep[4][MK];
            uint32_t cnt[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int m = 0; m < MK; ++m) keep[i][m] = 0xffffffffu;

            // prologue: block 0 -> buffer 0
            __syncthreads();
            for (int c = 0; c < my_pieces; ++c) {
                const int piece = threadIdx.x + 256 * c;
                if (piece < blk_pieces && piece / row_pieces < n) {
                    const int kr = piece / row_pieces, kc = piece % row_pieces;
                    *reinterpret_cast<uint4*>(kbuf + (kr * kstride) * ES + kc * 16) =
                        *reinterpret_cast<const uint4*>(Kg + static_cast<size_t>(kr) * dh * ES + kc * 16);
                }
            }
            __syncthreads();

            for (int blk = 0; blk < nblk; ++blk) {
                const int cur = blk & 1;
                // prefetch the next block into registers
                uint4 pre[4] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u),
                                make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
                const bool has_next = blk + 1 < nblk;
                if (has_next) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int piece = threadIdx.x + 256 * c;
                        if (c < my_pieces && piece < blk_pieces && (blk + 1) * KB + piece / row_pieces < n) {
                            const int kr = piece / row_pieces, kc = piece % row_pieces;
                            pre[c] = *reinterpret_cast<const uint4*>(
                                Kg + static_cast<size_t>((blk + 1) * KB + kr) * dh * ES + kc * 16);
                        }
                    }
                }
                const unsigned char* kb = kbuf + cur * KB * kstride * ES;
                float colv[KB / 16];
#pragma unroll
                for (int ct = 0; ct < KB / 16; ++ct) {
                    colv[ct] = 0.f;
                    if (blk * KB + ct * 16 >= n) continue;  // partial last block (n % 16 == 0)
                    Frag<STORE> B[DHS];
                    load_row_frags<STORE, DHS>(B, kb + (ct * 16 + r) * kstride * ES, g);
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s = 0; s < DHS; ++s) mma(A[s], B[s], acc);
                    const int key = blk * KB + ct * 16 + r;
                    const float knv = kn[key];
                    float cs = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = a.eps + fmaxf(qn_row[i] + knv - 2.f * acc[i], 0.f);
                        const uint32_t eb = __float_as_uint(e);
                        if (pass == 0 && (sel || stats || rowstat)) {
                            const float u = rv[i] ? fast_rcp(e) : 0.f;
                            zacc[i] += u;
                            if (rowstat) macc[i] = fmaf(u, lps[key], macc[i]);
                            if (sel && rv[i]) {
                                // keep the MK smallest of this lane, ascending
                                uint32_t x = eb;
#pragma unroll
                                for (int m = 0; m < MK; ++m) {
                                    const uint32_t lo = min(keep[i][m], x);
                                    x = max(keep[i][m], x);
                                    keep[i][m] = lo;
                                }
                            }
                        }
                        if (pass == 1) {
                            if (stats && rv[i]) cs = fmaf(fast_rcp(e), zinv[i], cs);
                            if (sel) {
                                const bool pred = rv[i] && eb <= tau[i];
                                const uint32_t m16 = static_cast<uint32_t>(ballot(pred) >> (16 * g)) & 0xffffu;
                                const uint32_t pos = cnt[i] + __popc(m16 & ((1u << r) - 1u));
                                if (pred && pos < static_cast<uint32_t>(a.cap)) {
                                    const size_t o = (static_cast<size_t>(bhh) * a.Tc + tw0 + 4 * g + i) * a.cap + pos;
                                    a.cand[o] = (static_cast<uint64_t>(eb) << 32) | static_cast<uint32_t>(key);
                                }
                                cnt[i] += __popc(m16);
                            }
                        }
                    }
                    colv[ct] = cs;
                }
                if (pass == 1 && stats) {
                    // sum over this wavefront's 16 tokens: across the four lane groups
#pragma unroll
                    for (int ct = 0; ct < KB / 16; ++ct) {
                        float x = colv[ct];
                        x += __shfl_xor(x, 16, 64);
                        x += __shfl_xor(x, 32, 64);
                        if (g == 0) colbuf[(cur * 4 + wave) * KB + ct * 16 + r] = x;
                    }
                }
                // stage the prefetched block into the other buffer
                if (has_next) {
                    unsigned char* nb = kbuf + (cur ^ 1) * KB * kstride * ES;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int piece = threadIdx.x + 256 * c;
                        if (c < my_pieces && piece < blk_pieces && (blk + 1) * KB + piece / row_pieces < n) {
                            const int kr = piece / row_pieces, kc = piece % row_pieces;
                            *reinterpret_cast<uint4*>(nb + (kr * kstride) * ES + kc * 16) = pre[c];
                        }
                    }
                }
                __syncthreads();
                if (pass == 1 && stats && threadIdx.x < KB && blk * KB + static_cast<int>(threadIdx.x) < n) {
                    // this tile's partial of pbar for the block's sub-keys, waves in order
                    const float* cb = colbuf + cur * 4 * KB + threadIdx.x;
                    const float s = ((cb[0] + cb[KB]) + cb[2 * KB]) + cb[3 * KB];
                    a.part[(static_cast<size_t>(bhh) * ntiles + tile) * n + blk * KB + threadIdx.x] = s;
                }
            }

            if (pass == 0) {
                // Z_t over the sixteen lanes that share token 4g+i
                float zt[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = zacc[i];
                    x += __shfl_xor(x, 1, 64);
                    x += __shfl_xor(x, 2, 64);
                    x += __shfl_xor(x, 4, 64);
                    x += __shfl_xor(x, 8, 64);
                    zt[i] = x;
                    zinv[i] = fast_rcp(x);
                }
                if (rowstat) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float x = macc[i];
                        x += __shfl_xor(x, 1, 64);
                        x += __shfl_xor(x, 2, 64);
                        x += __shfl_xor(x, 4, 64);
                        x += __shfl_xor(x, 8, 64);
                        if (r == 0 && rv[i]) {
                            const size_t o = static_cast<size_t>(bhh) * a.Tc + tw0 + 4 * g + i;
                            a.Z[o] = zt[i];
                            a.m[o] = x / zt[i];
                        }
                    }
                }
                if (sel) {
                    // tau = k'-th smallest of the 16*MK values kept by the token's lanes
                    constexpr int RS = (MK <= 1) ? 1 : (MK <= 2 ? 2 : 4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t v[RS];
#pragma unroll
                        for (int m = 0; m < RS; ++m) v[m] = (m < MK) ? keep[i][m] : 0xffffffffu;
                        bitonic_sort<RS, 16>(v);
                        const int kth = a.kh - 1;
                        uint32_t t = 0u;
#pragma unroll
                        for (int m = 0; m < RS; ++m)
                            if (m == kth / 16) t = v[m];
                        tau[i] = static_cast<uint32_t>(__shfl(static_cast<int>(t), 16 * g + (kth % 16), 64));
                    }
                }
            }
            if (last && sel && r == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (rv[i]) a.cnt[static_cast<size_t>(bhh) * a.Tc + tw0 + 4 * g + i] = static_cast<int32_t>(cnt[i]);
            }
        }
    }
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
            u[j] = 0x7f800000u;
            if (j < npl && i < n) {
                float d = 0.f;
                for (int x = 0; x < dh; ++x) {
                    const float diff = ld_elem<STORE>(q, x) - ld_elem<STORE>(K, kb + static_cast<size_t>(i) * dh + x);
                    d = fmaf(diff, diff, d);
                }
                u[j] = __float_as_uint(a.eps + d);
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
        out_e[lane] = __uint_as_float(static_cast<uint32_t>(key[0] >> 32));
        out_i[lane] = static_cast<int>(key[0] & 0xffffffffu);
    }
    wave_sync();
}

template <int R>
__device__ void product_topk(const SelectArgs& a, const float* e1, const int* i1, const float* e2, const int* i2,
                             int32_t* idx_out, float* w_out) {
    const int lane = lane_id();
    uint64_t key[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int c = r * 64 + lane;
        if (c < a.ncand) {
            const uint32_t ab = a.cand_ab.ab[c];
            const int ia = static_cast<int>(ab >> 6), ib = static_cast<int>(ab & 63u);
            const float P = e1[ia] * e2[ib];
            const uint32_t slot = static_cast<uint32_t>(i1[ia] * a.n + i2[ib]);
            key[r] = (static_cast<uint64_t>(__float_as_uint(P)) << 32) | slot;
        } else {
            key[r] = ~0ull;
        }
    }
    bitonic_sort<R, 64>(key);
    const float P = __uint_as_float(static_cast<uint32_t>(key[0] >> 32));
    const float P0 = __shfl(P, 0, 64);
    const float ratio = (lane < a.k) ? (P0 / P) : 0.f;
    const float sum = wave_sum(ratio);
    if (lane < a.k) {
        idx_out[lane] = static_cast<int32_t>(key[0] & 0xffffffffu);
        w_out[lane] = ratio / sum;
    }
}

template <int STORE>
__global__ __launch_bounds__(256) void k_select(SelectArgs a) {
    __shared__ uint64_t buf[4][64];
    __shared__ uint32_t hist[4][256];
    __shared__ float se[4][2][kMaxKHalf];
    __shared__ int si[4][2][kMaxKHalf];
    const int wave = threadIdx.x >> 6;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + wave;  // over B*Tc*H
    if (item >= static_cast<int64_t>(a.B) * a.Tc * a.H) return;
    const int h = static_cast<int>(item % a.H);
    const int64_t bt = item / a.H;
    const int t = static_cast<int>(bt % a.Tc), b = static_cast<int>(bt / a.Tc);
    for (int half = 0; half < 2; ++half)
        half_topk<STORE>(a, b, t, h, half, hist[wave], buf[wave], se[wave][half], si[wave][half]);
    const size_t o = static_cast<size_t>(b) * a.iw_bstride + (static_cast<size_t>(t) * a.H + h) * a.k;
    if (a.ncand <= 64) product_topk<1>(a, se[wave][0], si[wave][0], se[wave][1], si[wave][1], a.idx + o, a.w + o);
    else if (a.ncand <= 128) product_topk<2>(a, se[wave][0], si[wave][0], se[wave][1], si[wave][1], a.idx + o, a.w + o);
    else product_topk<4>(a, se[wave][0], si[wave][0], se[wave][1], si[wave][1], a.idx + o, a.w + o);
}

template <int STORE, int DHS, int MK>
hipError_t score_t(const ScoreArgs& a, hipStream_t s) {
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int KB = kKB<STORE>;
    const size_t lds = static_cast<size_t>(2) * KB * (a.dh + 16 / ES) * ES + 2 * 4 * KB * 4 +
                       ((a.mode & kScoreRowStat) ? static_cast<size_t>(a.n) * 4 : 0);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_score<STORE, DHS, MK>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int ntiles = (a.Tc + kTok - 1) / kTok;
    const unsigned grid = static_cast<unsigned>(a.B) * a.H * ntiles;
    hipLaunchKernelGGL((k_score<STORE, DHS, MK>), dim3(grid), dim3(256), lds, s, a);
    return hipGetLastError();
}

template <int STORE, int DHS>
hipError_t score_mk(const ScoreArgs& a, hipStream_t s) {
    switch (score_keep(a.kh)) {
        case 2: return score_t<STORE, DHS, 2>(a, s);
        case 3: return score_t<STORE, DHS, 3>(a, s);
        case 4: return score_t<STORE, DHS, 4>(a, s);
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

hipError_t launch_score(const ScoreArgs& a, int store, hipStream_t s) {
    return store == kBF16 ? score_s<kBF16>(a, s) : score_s<kF32>(a, s);
}

hipError_t launch_select(const SelectArgs& a, int store, hipStream_t s) {
    const int64_t items = static_cast<int64_t>(a.B) * a.Tc * a.H;
    const unsigned grid = static_cast<unsigned>((items + 3) / 4);
    if (store == kBF16) hipLaunchKernelGGL(k_select<kBF16>, dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_select<kF32>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace fwpkm
