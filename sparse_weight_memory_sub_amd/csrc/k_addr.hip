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
// wavefront owns 16 keys and walks the chunk's tokens in blocks of 32.  Each
// block's query rows (d_h-contiguous) are staged in LDS by direct
// global-to-LDS loads, double-buffered; for fp32 storage also the same rows
// transposed (token-contiguous, written once per chunk in tiles of qt_tile).
// Per block:
//  1. recompute the 32x16 distance tile on the matrix cores (same operands,
//     order and roundings as the scoring sweep, so the values are bitwise
//     the same);
//  2. form a_ti for its keys;
//  3. accumulate sum_t a_ti q_t on the matrix cores (keys x tokens times
//     tokens x d_h; for bf16 storage the tokens x d_h operand comes from the
//     query tile itself through gfx950's transposing LDS reads, and a_ti is
//     split into a bf16 high part and a bf16 low part, two MFMAs, about 16
//     bits of a_ti; for fp32 from the transposed tile).
// Then K_i <- K_i - lr (sum_t a_ti q_t - (sum_t a_ti) K_i), rounded to the
// storage type, and ||K_i||^2 of the stored key is written for the next
// chunk's scoring.  Every key is read and written by one wavefront only.
#include "mfma_frag.h"

namespace fwpkm {

namespace {

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


// The chunk's transposed query halves in a launch of their own, one 64 x 64
// tile per 256-thread workgroup (the scoring path, whose row-statistic
// workgroups are too large and hold too much LDS to carry these tiles well).
template <int STORE>
__global__ __launch_bounds__(256) void k_qt(QtArgs a) {
    __shared__ __align__(16) unsigned char tile[qt_tile_bytes<STORE>()];
    qt_tile<STORE, 4>(a, blockIdx.x, blockIdx.y, blockIdx.z, tile);
}

// Split partials: [B*H*2][split][n][dh] sums over the split's tokens of
// a_ti q_t, then [B*H*2][split][n] sums of a_ti.
__device__ __forceinline__ float* part_colsum(const KgradArgs& a, int dh) {
    return a.part + static_cast<size_t>(a.B) * a.H * 2 * a.split * a.n * dh;
}

// Key update of one wave's 16 keys from the summed tiles: gacc[c][i] holds
// sum_t a_ti q_t[16c + r] of key key0 + 4g + i, colsum (lanes r) sum_t a_ti
// of key key0 + r.  IDW: K -= lr * (sum a q - (sum a) K); dot: K -= lr * sum a q.
// Rewrites ||K||^2 of the new keys.
template <int STORE, int DHS, bool DOT>
__device__ __forceinline__ void kgrad_apply(const KgradArgs& a, unsigned char* Kb, int bhh, int key0, int r, int g,
                                            const f32x4_t* gacc, float colsum) {
    constexpr int DH = 32 * DHS;
    constexpr int NCT = DHS * 2;
    const int n = a.n;
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
            const size_t off = static_cast<size_t>(k) * DH + col;
            const float kv = ld_elem<STORE>(Kb, off);
            const float grad = DOT ? gacc[c][i] : gacc[c][i] - cs[i] * kv;
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

template <int STORE, int DHS, bool DOT, bool SPLIT>
__global__ __launch_bounds__(256, 3) void k_kgrad(KgradArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int DH = 32 * DHS;
    constexpr int CPRQ = DH * ES / 16;        // chunks per query row (wide image, 32 rows)
    constexpr int CPRT = 32 * ES / 16;        // chunks per transposed row (narrow image, DH rows)
    constexpr int QB = 32 * CPRQ * 16;        // bytes of one query tile
    constexpr int QBUF = QB + 3 * 32 * 4;     // a query tile + qn, 1/Z, m of its 32 tokens
    // bf16: the sum over tokens takes its query operand from the query tile
    // itself by transposing LDS reads; fp32: from a transposed tile
    constexpr bool TR = STORE == kBF16;
    const int n = a.n, H = a.H, Tc = a.Tc;

    const int nkb = (n + 63) / 64;
    const uint32_t lid = xcd_remap(blockIdx.x, gridDim.x);
    const int kb = static_cast<int>(lid % nkb);
    const int split = SPLIT ? a.split : 1;
    const int sp = static_cast<int>((lid / nkb) % split);
    const int bhh = static_cast<int>(lid / nkb / split);  // (b*H + h)*2 + half
    const int half = bhh & 1, bh = bhh >> 1;
    const int h = bh % H, b = bh / H;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int key0 = kb * 64 + wave * 16;
    const bool active = key0 < n;
    const int key = key0 + r;
    unsigned char* Kb = static_cast<unsigned char*>(half ? a.K2 : a.K1) + static_cast<size_t>(bh) * n * DH * ES;
    const unsigned char* qbase = static_cast<const unsigned char*>(a.q) +
        (static_cast<size_t>(b) * a.q_bstride + h * 2 * DH + half * DH) * ES;
    const uint32_t qstride = static_cast<uint32_t>(H * 2 * DH * ES);
    const unsigned char* tbase = static_cast<const unsigned char*>(a.qT) + static_cast<size_t>(bhh) * DH * a.Tp * ES;
    const uint32_t tstride = static_cast<uint32_t>(a.Tp * ES);

    // this wave's 16 keys as the B operand of the distance tiles, scaled by -2
    Frag<STORE> Bk[DHS];
    float kn = 0.f, lpv = 0.f;
    if (active) {
        load_row_frags<STORE, DHS>(Bk, Kb + static_cast<size_t>(key) * DH * ES, g);
        if constexpr (!DOT) {
#pragma unroll
            for (int s = 0; s < DHS; ++s) frag_scale_m2(Bk[s]);
            kn = a.knorm[static_cast<size_t>(bhh) * n + key];
        }
        lpv = a.lp[static_cast<size_t>(bhh) * n + key];
    }
    const int eps_bits = __float_as_int(a.eps);
    const FragBase<STORE, DHS> fq(r, g);
    // transposed-tile offsets of the operand column d = 16c + r: tokens 4g..4g+3
    // and 16+4g..16+4g+3 of the block, adjacent in the qt_tile order (one 16-byte
    // chunk for bf16, two for fp32)
    uint32_t tb0 = 0, tb1 = 0;
    // bf16, by transposing reads of the query tile: a read hands lane r of a
    // 16-lane group component r % 4 of the 8 bytes addressed by lanes
    // r / 4, 4 + r / 4, 8 + r / 4 and 12 + r / 4.  So lane m of group g
    // addresses columns 16c + 4(m % 4) .. +3 of token row 4g + m / 4 (and
    // of row 16 + 4g + m / 4), and lane r receives column 16c + r of tokens
    // 4g..4g+3 (16+4g..16+4g+3): the eight k-elements of the a_ti fragment,
    // in its order.  Column chunk 2c + (m % 4) / 2 of a row R sits at chunk
    // position (2c + (m % 4) / 2) ^ swz(R) = 2c ^ tk (the image's swizzle).
    uint32_t trow1 = 0, trow2 = 0;
    int tk1 = 0, tk2 = 0;
    if constexpr (TR) {
        const int R1 = 4 * g + (r >> 2), R2 = R1 + 16, u = r & 3;
        trow1 = static_cast<uint32_t>(R1 * CPRQ * 16 + (u & 1) * 8);
        trow2 = static_cast<uint32_t>(R2 * CPRQ * 16 + (u & 1) * 8);
        tk1 = (u >> 1) ^ swz<CPRQ>(R1);
        tk2 = (u >> 1) ^ swz<CPRQ>(R2);
    } else {
        const int f = swz<CPRT, true>(r);
        tb0 = static_cast<uint32_t>(r * CPRT + ((2 * g) ^ f)) * 16u;
        tb1 = static_cast<uint32_t>(r * CPRT + ((2 * g + 1) ^ f)) * 16u;
    }

    constexpr int NCT = DHS * 2;  // 16-wide column tiles of d_h
    f32x4_t gacc[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) gacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float colsum = 0.f;
    // a_ti = (2/C)(ln pbar_i - m_t)/(Z_t e^2) for IDW, (1/C)(ln pbar_i - m_t) e^(s - M_t)/Z_t for dot
    const float inv_tc2 = (DOT ? 1.f : 2.f) / static_cast<float>(Tc);

    // Token blocks of 32; this workgroup takes blocks b0 .. b0+nblk-1 of the
    // chunk (all of them without a split).  Key blocks of one (sequence, head,
    // half) run side by side and read the same query rows: each starts at a
    // different block (fixed order per key block, so the sums stay
    // reproducible).
    const int b0 = SPLIT ? sp * a.per : 0;
    const int nblk = SPLIT ? min(a.per, (Tc + 31) / 32 - b0) : (Tc + 31) / 32;
    auto tok_block = [&](int bi) { return (b0 + (bi + kb) % nblk) * 32; };
    // LDS: two query tiles (with their token statistics), used in turn, and
    // (fp32) one transposed tile
    unsigned char* tbuf = smem + 2 * QBUF;
    auto stage_q = [&](unsigned char* buf, int tb) {
        const int nv = Tc - tb;
        dma_rows<CPRQ, 32, 4, false>(buf, qbase + static_cast<size_t>(tb) * qstride, qstride, nv, wave, lane);
        if constexpr (TR) {
            // the rows past the chunk hold zeros: the transposing reads hand
            // them to the sum over tokens, whose a_ti are 0 there
            if (nv < 32)
                for (int i = static_cast<int>(threadIdx.x); i < (32 - nv) * CPRQ; i += 256)
                    *reinterpret_cast<uint4*>(buf + (static_cast<size_t>(nv) * CPRQ + i) * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto stage_t = [&](int tb) {
        if constexpr (!TR)
            dma_rows<CPRT, DH, 4, true>(tbuf, tbase + static_cast<size_t>(tb) * ES, tstride, DH, wave, lane);
    };
    // qn, 1/Z, m of tokens tb..tb+31 (zeros past the chunk), threads 0..95
    auto tq_load = [&](int tb) {
        float x = 0.f;
        if (threadIdx.x < 96) {
            const int which = threadIdx.x >> 5, t = tb + (threadIdx.x & 31);
            if (t < Tc) {
                const size_t o = static_cast<size_t>(bhh) * Tc + t;
                // first row: ||q||^2 (IDW) or the row maximum M_t of s (dot)
                x = which == 0 ? (DOT ? a.M[o] : a.qn[o]) : (which == 1 ? __builtin_amdgcn_rcpf(a.Z[o]) : a.m[o]);
            }
        }
        return x;
    };
    auto tq_store = [&](unsigned char* buf, float x) {
        if (threadIdx.x < 96) reinterpret_cast<float*>(buf + QB)[threadIdx.x] = x;
    };

    stage_q(smem, tok_block(0));
    stage_t(tok_block(0));
    tq_store(smem, tq_load(tok_block(0)));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Per block: the next query tile is requested first; the distance tile
    // uses the current one; once every wave's part of the transposed tile
    // has landed (barrier 1) the sum over tokens reads it; after barrier 2
    // the next transposed tile is requested, to land under the next block's
    // distance recompute.
    for (int bi = 0; bi < nblk; ++bi) {
        unsigned char* cur = smem + (bi & 1) * QBUF;
        unsigned char* nxt = smem + ((bi + 1) & 1) * QBUF;
        const int tb = tok_block(bi);
        float tqn = 0.f;
        if (bi + 1 < nblk) {
            stage_q(nxt, tok_block(bi + 1));
            tqn = tq_load(tok_block(bi + 1));
        }
        float av[8];  // a_ti of this wave's keys for the block's tokens
        if (active) {
            const float* tq = reinterpret_cast<const float*>(cur + QB);
            // the two 16-token halves' distance tiles side by side: two
            // independent accumulation chains, each in k-block order
            f32x4_t accs[2];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int i = 0; i < 4; ++i) accs[sub][i] = kn;
#pragma unroll
            for (int s = 0; s < DHS; ++s) {
                Frag<STORE> A0, A1;
                lds_frag<STORE, DHS>(A0, cur, fq, 0, s);
                lds_frag<STORE, DHS>(A1, cur, fq, 1, s);
                mma(A0, Bk[s], accs[0]);
                mma(A1, Bk[s], accs[1]);
            }
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                const f32x4_t acc = accs[sub];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = sub * 16 + 4 * g + i;
                    float val;
                    if constexpr (DOT) {
                        val = inv_tc2 * (lpv - tq[64 + row]) * tq[32 + row] * __expf(acc[i] - tq[row]);
                    } else {
                        const float e = __int_as_float(max(__float_as_int((tq[row] + a.eps) + acc[i]), eps_bits));
                        const float ie = __builtin_amdgcn_rcpf(e);
                        val = inv_tc2 * (lpv - tq[64 + row]) * tq[32 + row] * ie * ie;
                    }
                    // tokens past the chunk have 1/Z = 0; the select also drops
                    // whatever their (unfilled) query rows produced
                    av[sub * 4 + i] = (tb + row < Tc) ? val : 0.f;
                    colsum += av[sub * 4 + i];
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's parts of the next query tile (and the transposed tile) have landed
        __syncthreads();
        if (active) {
            // sum_t a_ti q_t: keys x tokens (A) times tokens x d_h (B)
            if constexpr (STORE == kBF16) {
                Frag<kBF16> Ahi, Alo;
                uint32_t hi[4], lo[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    hi[j] = pack_bf16x2(av[2 * j], av[2 * j + 1]);
                    lo[j] = pack_bf16x2(av[2 * j] - __uint_as_float(hi[j] << 16),
                                        av[2 * j + 1] - __uint_as_float(hi[j] & 0xffff0000u));
                }
                Ahi.v = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
                Alo.v = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
                // four column tiles at a time: their operands requested
                // together, then the high parts, then the low parts (each
                // accumulator still takes high before low)
                constexpr int G = NCT % 4 == 0 ? 4 : 1;
                // the read offsets are formed per block (two operations each),
                // not kept in registers across the loop (the kernel has none
                // to spare at three workgroups per compute unit)
                asm volatile("" : "+v"(tk1), "+v"(trow1));
#pragma unroll
                for (int c0 = 0; c0 < NCT; c0 += G) {
                    Frag<kBF16> Bq[G];
#pragma unroll
                    for (int j = 0; j < G; ++j) {
                        const int c = c0 + j;
                        const uint32_t o1 = trow1 + (static_cast<uint32_t>((2 * c) ^ tk1) << 4);
                        // rows 16 on: the same swizzle when rows hold 16 or more chunks
                        const uint32_t o2 = (CPRQ >= 16) ? o1 + 16u * CPRQ * 16u
                                                         : trow2 + (static_cast<uint32_t>((2 * c) ^ tk2) << 4);
                        const v4i16_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) v4i16_t*)(cur + o1));
                        const v4i16_t x2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) v4i16_t*)(cur + o2));
                        const uint2 w1 = __builtin_bit_cast(uint2, x1), w2 = __builtin_bit_cast(uint2, x2);
                        Bq[j].v = u32x4_t{w1.x, w1.y, w2.x, w2.y};
                    }
#pragma unroll
                    for (int j = 0; j < G; ++j) mma(Ahi, Bq[j], gacc[c0 + j]);
#pragma unroll
                    for (int j = 0; j < G; ++j) mma(Alo, Bq[j], gacc[c0 + j]);
                }
            } else {
                Frag<kF32> A;
#pragma unroll
                for (int j = 0; j < 8; ++j) A.v[j] = av[j];
#pragma unroll
                for (int c = 0; c < NCT; ++c) {
                    const unsigned char* tp = tbuf + static_cast<uint32_t>(c * 16 * CPRT * 16);
                    const float4 x0 = *reinterpret_cast<const float4*>(tp + tb0);
                    const float4 x1 = *reinterpret_cast<const float4*>(tp + tb1);
                    Frag<kF32> Bq;
                    Bq.v[0] = x0.x; Bq.v[1] = x0.y; Bq.v[2] = x0.z; Bq.v[3] = x0.w;
                    Bq.v[4] = x1.x; Bq.v[5] = x1.y; Bq.v[6] = x1.z; Bq.v[7] = x1.w;
                    mma(A, Bq, gacc[c]);
                }
            }
        }
        if (bi + 1 < nblk) tq_store(nxt, tqn);
        __syncthreads();  // every wave is done with the transposed tile
        if (bi + 1 < nblk) stage_t(tok_block(bi + 1));
    }
    if (!active) return;

    // colsum over the four lane groups: lanes with the same r hold the same key
    colsum += __shfl_xor(colsum, 16, 64);
    colsum += __shfl_xor(colsum, 32, 64);
    if constexpr (SPLIT) {
        // leave this split's sums for k_kgrad_finish, one row of d_h per key
        const size_t rows = static_cast<size_t>(bhh) * a.split + sp;
        float* pg = a.part + rows * n * DH;
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
#pragma unroll
            for (int i = 0; i < 4; ++i) pg[static_cast<size_t>(key0 + 4 * g + i) * DH + 16 * c + r] = gacc[c][i];
        }
        if (g == 0) part_colsum(a, DH)[rows * n + key0 + r] = colsum;
    } else {
        kgrad_apply<STORE, DHS, DOT>(a, Kb, bhh, key0, r, g, gacc, colsum);
    }
}

// Split sums and key update of 8 columns (8j .. 8j+7) of key kg (bhh*n + key);
// the new values also go to out[0..7].
template <int STORE, int DHS, bool DOT>
__device__ __forceinline__ void update_row(const KgradArgs& a, size_t kg, int j, float* out) {
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int DH = 32 * DHS;
    const int n = a.n;
    const int bhh = static_cast<int>(kg / n), k = static_cast<int>(kg % n);
    const int bh = bhh >> 1, half = bhh & 1;
    const float* pg = a.part + (static_cast<size_t>(bhh) * a.split * n + k) * DH + 8 * j;
    const float* pc = part_colsum(a, DH) + static_cast<size_t>(bhh) * a.split * n + k;
    const size_t sstride = static_cast<size_t>(n) * DH;
    // every split's partials requested first (at most kKgradMaxSplit), then
    // added in split order
    float4 x0[kKgradMaxSplit], x1[kKgradMaxSplit];
    float xc[kKgradMaxSplit];
#pragma unroll
    for (int sp = 0; sp < kKgradMaxSplit; ++sp) {
        const int q = sp < a.split ? sp : 0;
        x0[sp] = *reinterpret_cast<const float4*>(pg + q * sstride);
        x1[sp] = *reinterpret_cast<const float4*>(pg + q * sstride + 4);
        xc[sp] = pc[static_cast<size_t>(q) * n];
    }
    float4 s0 = x0[0], s1 = x1[0];
    float cs = xc[0];
#pragma unroll
    for (int sp = 1; sp < kKgradMaxSplit; ++sp) {
        if (sp < a.split) {
            s0.x += x0[sp].x; s0.y += x0[sp].y; s0.z += x0[sp].z; s0.w += x0[sp].w;
            s1.x += x1[sp].x; s1.y += x1[sp].y; s1.z += x1[sp].z; s1.w += x1[sp].w;
            cs += xc[sp];
        }
    }
    const float gs[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    unsigned char* Kb = static_cast<unsigned char*>(half ? a.K2 : a.K1) +
        (static_cast<size_t>(bh) * n * DH + static_cast<size_t>(k) * DH + 8 * j) * ES;
    float kv[8], kn[8];
    if constexpr (STORE == kBF16) {
        const uint4 x = *reinterpret_cast<const uint4*>(Kb);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kv[2 * e] = __uint_as_float(w[e] << 16);
            kv[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    } else {
        const float4 x0 = reinterpret_cast<const float4*>(Kb)[0], x1 = reinterpret_cast<const float4*>(Kb)[1];
        kv[0] = x0.x; kv[1] = x0.y; kv[2] = x0.z; kv[3] = x0.w;
        kv[4] = x1.x; kv[5] = x1.y; kv[6] = x1.z; kv[7] = x1.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // IDW: sum_t a (q_t - K_i); dot: sum_t a q_t
        const float grad = DOT ? gs[e] : gs[e] - cs * kv[e];
        float x = kv[e] - a.lr * grad;
        if constexpr (STORE == kBF16) x = bf16_to_f32(f32_to_bf16(x));
        kn[e] = x;
        out[e] = x;
    }
    if constexpr (STORE == kBF16) {
        uint4 y;
        y.x = pack_bf16x2(kn[0], kn[1]);
        y.y = pack_bf16x2(kn[2], kn[3]);
        y.z = pack_bf16x2(kn[4], kn[5]);
        y.w = pack_bf16x2(kn[6], kn[7]);
        *reinterpret_cast<uint4*>(Kb) = y;
    } else {
        reinterpret_cast<float4*>(Kb)[0] = make_float4(kn[0], kn[1], kn[2], kn[3]);
        reinterpret_cast<float4*>(Kb)[1] = make_float4(kn[4], kn[5], kn[6], kn[7]);
    }
}

// Sum over the token splits of k_kgrad, in split order, then the key update:
// one thread per 8 columns of a key, DH/8 adjacent threads per key.  The new
// norms are summed in k_knorm's order (lane r over columns r + 16c, then
// across the 16 lanes), so a run that recomputes them from the keys agrees
// bit for bit with one that carries them.
template <int STORE, int DHS, bool DOT>
__global__ __launch_bounds__(256) void k_kgrad_finish(KgradArgs a) {
    constexpr int DH = 32 * DHS;
    constexpr int TPK = DH / 8;   // threads per key: 4 .. 32
    constexpr int KPW = 256 / TPK;  // keys per workgroup
    __shared__ float rows[256 * 8];  // the workgroup's new keys, row-major
    const int n = a.n;
    const size_t total = static_cast<size_t>(a.B) * a.H * 2 * n;
    const size_t t = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    const size_t kg = t / TPK;  // (bhh * n) + key
    const int j = static_cast<int>(t % TPK);
    if (kg < total) update_row<STORE, DHS, DOT>(a, kg, j, rows + threadIdx.x * 8);
    __syncthreads();
    for (int pr = threadIdx.x; pr < KPW * 16; pr += 256) {  // uniform per wave
        const int kl = pr >> 4, r = pr & 15;
        float x = 0.f;
#pragma unroll
        for (int c = 0; c < DH / 16; ++c) {
            const float v = rows[kl * DH + 16 * c + r];
            x = fmaf(v, v, x);
        }
        x += __shfl_xor(x, 1, 64);
        x += __shfl_xor(x, 2, 64);
        x += __shfl_xor(x, 4, 64);
        x += __shfl_xor(x, 8, 64);
        const size_t key = static_cast<size_t>(blockIdx.x) * KPW + kl;
        if (r == 0 && key < total) a.knorm[key] = x;
    }
}


template <int STORE, int DHS, bool DOT>
hipError_t kgrad_t(const KgradArgs& a, hipStream_t s) {
    constexpr int ES = Store<STORE>::kBytes;
    constexpr int DH = 32 * DHS;
    // two query tiles with their token statistics, and for fp32 the transposed tile
    constexpr size_t LDS = 2 * (static_cast<size_t>(32) * DH * ES + 3 * 32 * 4) +
                           (STORE == kF32 ? static_cast<size_t>(DH) * 32 * ES : 0);
    static bool attr_set = false;
    if (!attr_set) {
        for (const void* f : {reinterpret_cast<const void*>(&k_kgrad<STORE, DHS, DOT, false>),
                              reinterpret_cast<const void*>(&k_kgrad<STORE, DHS, DOT, true>)}) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
            if (e != hipSuccess) return e;
        }
        attr_set = true;
    }
    const int nkb = (a.n + 63) / 64;
    const unsigned grid = static_cast<unsigned>(a.B) * a.H * 2 * nkb;
    if (a.split <= 1) {
        hipLaunchKernelGGL((k_kgrad<STORE, DHS, DOT, false>), dim3(grid), dim3(256), LDS, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((k_kgrad<STORE, DHS, DOT, true>), dim3(grid * a.split), dim3(256), LDS, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t threads = static_cast<size_t>(a.B) * a.H * 2 * a.n * (DH / 8);
    hipLaunchKernelGGL((k_kgrad_finish<STORE, DHS, DOT>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int STORE>
hipError_t kgrad_s(const KgradArgs& a, hipStream_t s) {
    switch (a.dh / 32) {
        case 1: return a.dot ? kgrad_t<STORE, 1, true>(a, s) : kgrad_t<STORE, 1, false>(a, s);
        case 2: return a.dot ? kgrad_t<STORE, 2, true>(a, s) : kgrad_t<STORE, 2, false>(a, s);
        case 4: return a.dot ? kgrad_t<STORE, 4, true>(a, s) : kgrad_t<STORE, 4, false>(a, s);
        case 8: return a.dot ? kgrad_t<STORE, 8, true>(a, s) : kgrad_t<STORE, 8, false>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

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

hipError_t launch_qt(const QtArgs& a, int store, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((a.Tp + 63) / 64), static_cast<unsigned>((a.dh + 63) / 64),
                    static_cast<unsigned>(a.B * a.H * 2));
    if (store == kBF16) hipLaunchKernelGGL(k_qt<kBF16>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_qt<kF32>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace fwpkm
