// fwpkm_internal.h -- device helpers, kernel argument blocks and launch
// entry points shared by the gfx950 HIP sources of the FwPKM library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace fwpkm {

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------
enum : int { kF32 = 0, kBF16 = 1 };

template <int STORE> struct Store;
template <> struct Store<kF32> {
    using T = float;
    static constexpr int kBytes = 4;
};
template <> struct Store<kBF16> {
    using T = uint16_t;
    static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Value of lane (lane ^ m) of a wavefront, for a stride m known at compile
// time after unrolling: data-parallel-primitive moves inside a 16-lane row
// for m = 1, 2, 4, 8 (quad permutes and row rotates; row_ror:n reads lane
// (i - n) mod 16), a bit-mask swizzle for 16, a permute through the LDS
// crossbar otherwise.
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int m) {
    const int v = static_cast<int>(x);
    switch (m) {
        case 1: return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
        case 2: return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
        case 4: {
            const int down = __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false);  // lane i - 4
            const int up = __builtin_amdgcn_mov_dpp(v, 0x12C, 0xF, 0xF, false);    // lane i + 4
            return static_cast<uint32_t>((__lane_id() & 4) ? down : up);
        }
        case 8: return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false));
        case 16: return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(v, 0x401F));
        default: return static_cast<uint32_t>(__shfl_xor(v, m, 64));
    }
}
__device__ __forceinline__ float xor_lane(float x, int m) {
    return __uint_as_float(xor_lane(__float_as_uint(x), m));
}

// 16-byte global load / store; NT marks it non-temporal (streamed data that
// should not displace reused lines from the caches).
typedef __attribute__((ext_vector_type(4))) unsigned int nt_u32x4;
template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
    if constexpr (NT) {
        const nt_u32x4 v = __builtin_nontemporal_load(static_cast<const nt_u32x4*>(p));
        return make_uint4(v[0], v[1], v[2], v[3]);
    } else {
        return *static_cast<const uint4*>(p);
    }
}
template <bool NT>
__device__ __forceinline__ void st16(void* p, uint4 v) {
    if constexpr (NT) {
        const nt_u32x4 x = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(x, static_cast<nt_u32x4*>(p));
    } else {
        *static_cast<uint4*>(p) = v;
    }
}

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((ext_vector_type(2))) float f2_t;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf2_t;
    const f2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2_t));
}

template <int STORE> __device__ __forceinline__ float ld_elem(const void* p, size_t i);
template <> __device__ __forceinline__ float ld_elem<kF32>(const void* p, size_t i) {
    return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float ld_elem<kBF16>(const void* p, size_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <int STORE> __device__ __forceinline__ void st_elem(void* p, size_t i, float x);
template <> __device__ __forceinline__ void st_elem<kF32>(void* p, size_t i, float x) {
    static_cast<float*>(p)[i] = x;
}
template <> __device__ __forceinline__ void st_elem<kBF16>(void* p, size_t i, float x) {
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16(x));
}

// Load 8 consecutive storage elements (16 B for bf16, 32 B for f32) as floats.
template <int STORE> __device__ __forceinline__ void ld8(const void* p, size_t i, float (&x)[8]);
template <> __device__ __forceinline__ void ld8<kF32>(const void* p, size_t i, float (&x)[8]) {
    const float4* s = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    float4 a = s[0], b = s[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <> __device__ __forceinline__ void ld8<kBF16>(const void* p, size_t i, float (&x)[8]) {
    uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + i);
    x[0] = __uint_as_float(a.x << 16); x[1] = __uint_as_float(a.x & 0xffff0000u);
    x[2] = __uint_as_float(a.y << 16); x[3] = __uint_as_float(a.y & 0xffff0000u);
    x[4] = __uint_as_float(a.z << 16); x[5] = __uint_as_float(a.z & 0xffff0000u);
    x[6] = __uint_as_float(a.w << 16); x[7] = __uint_as_float(a.w & 0xffff0000u);
}

// ---------------------------------------------------------------------------
// wavefront helpers (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Orders LDS traffic of one wavefront: everything before is visible after.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Order-preserving map of floats to unsigned ints (ascending float ->
// ascending uint) and its inverse: dot scores select on ord(-s).
__device__ __forceinline__ uint32_t ord_f32(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord_f32(uint32_t u) {
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// ln pbar_i = ln((sum over the tiles, in order, of part[tile][i]) / Tc):
// the usage marginal of sub-key i from its per-tile partial sums.
__device__ __forceinline__ float log_pbar(const float* part, int ntiles, int n, int i, int Tc) {
    float s = 0.f;
    for (int t = 0; t < ntiles; ++t) s += part[static_cast<size_t>(t) * n + i];
    return logf(s / static_cast<float>(Tc));
}

// The median of a, b, c, written so that the compiler emits one v_med3_u32.
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
    return max(min(a, b), min(max(a, b), c));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += xor_lane(x, o);
    return x;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
    const int l = lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (l >= o) x += y;
    }
    return x;
}

// Map the hardware-linear workgroup id to a logical id so that the
// workgroups the dispatcher sends to one XCD (linear id mod 8) receive a
// contiguous range of logical ids: neighbouring tiles then share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t lin, uint32_t total) {
    const uint32_t nx = 8;
    const uint32_t x = lin % nx, i = lin / nx;
    const uint32_t q = total / nx, r = total % nx;
    return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// ---------------------------------------------------------------------------
// kernel argument blocks
// ---------------------------------------------------------------------------
constexpr int kMaxCand = 256;   // product candidates per (token, head)
constexpr int kMaxKHalf = 64;
constexpr int kMaxK = 64;

// Candidate pairs (a, b) of the two sorted top-k' lists that can reach the
// final top-k: (a+1)(b+1) <= k.  Packed a*64 + b.
struct CandTable {
    uint16_t ab[kMaxCand];
};

enum ScoreMode : int {
    kScoreSelect = 1,   // candidate lists of the per-half top-k' -> cand, cnt
    kScoreStats = 2,    // per-tile partial sums of p over tokens -> part
    kScoreRowStat = 4,  // Z_t and m_t = sum_i p_ti log pbar_i -> Z, m
    kScoreRows = 8,     // every e_ti written out -> erow
};
constexpr int kRowTok = 16;  // chunks this short are always scored by whole rows
// Tokens per scoring workgroup, 16 per wavefront: 64, 128 or 256, chosen
// per launch by score_tile().
constexpr int kScoreTokMin = 64;
constexpr int kGatherPart = 16;         // gather: entries summed per part (parts added in order)
constexpr int kGatherSplitBelow = 1024; // gather: one wavefront per part below this many tokens
constexpr int kScoreTokMax = 256;

// Transposed query halves of a chunk, qT[bhh][d][t'] for t' < Tp (Tp = Tc
// rounded up to 32; zeros past Tc), the token-contiguous operand of the sum
// over tokens in the key step.  Within each 32-token block the tokens are
// stored in groups of four in the order 0, 4, 1, 5, 2, 6, 3, 7 (group j =
// tokens 4j..4j+3), so that tokens 4g..4g+3 and 16+4g..16+4g+3 -- the eight
// k-elements lane group g of an MFMA operand holds -- are adjacent.  64x64
// tiles through LDS, one per workgroup of 256 or 1024 threads: tile (bx, by) of
// (tokens, d) of query half bz = (b*H + h)*2 + half.
struct QtArgs {
    const void* q;        // token t of sequence b at q + b*q_bstride + t*H*2*dh
    int64_t q_bstride;
    void* qT;             // [B][H][2][dh][Tp]
    int B, Tc, Tp, H, dh;
};

__host__ __device__ constexpr int qt_pos(int t) {
    const int blk = t & ~31, grp = (t >> 2) & 7;
    return blk + (((grp & 3) << 1) | (grp >> 2)) * 4 + (t & 3);
}

template <int STORE>
__host__ __device__ constexpr int qt_tile_bytes() {
    return 64 * 65 * Store<STORE>::kBytes;
}

// Tiles of the transposed queries: (tokens, d) tiles x bz.
inline int64_t qt_tiles(const QtArgs& a) {
    return static_cast<int64_t>((a.Tp + 63) / 64) * ((a.dh + 63) / 64) * a.B * a.H * 2;
}

template <int STORE, int GROUPS>
__device__ __forceinline__ void qt_tile(const QtArgs& a, int bx, int by, int bz, unsigned char* lds) {
    using E = typename Store<STORE>::T;
    static_assert(GROUPS == 4 || GROUPS == 16, "256 or 1024 threads");
    constexpr int PER = 64 / GROUPS;  // rows of the tile per 64-thread group
    E (*tile)[65] = reinterpret_cast<E (*)[65]>(lds);
    const int t0 = bx * 64, d0 = by * 64;
    const int bhh = bz;
    const int half = bhh & 1, bh = bhh >> 1;
    const int h = bh % a.H, b = bh / a.H;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const E* q = static_cast<const E*>(a.q) + static_cast<size_t>(b) * a.q_bstride + h * 2 * a.dh + half * a.dh;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int tl = ty * PER + i, t = t0 + tl, d = d0 + tx;
        E v{};
        if (t < a.Tc && d < a.dh) v = q[static_cast<size_t>(t) * a.H * 2 * a.dh + d];
        tile[tl][tx] = v;
    }
    __syncthreads();
    E* out = static_cast<E*>(a.qT) + static_cast<size_t>(bhh) * a.dh * a.Tp;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int dl = ty * PER + i, d = d0 + dl, t = t0 + tx;
        if (d < a.dh && t < a.Tp) out[static_cast<size_t>(d) * a.Tp + qt_pos(t)] = tile[tx][dl];
    }
}

// Linear tile index -> (bx, by, bz) of qt_tile.
template <int STORE, int GROUPS>
__device__ __forceinline__ void qt_tile_linear(const QtArgs& a, int64_t i, unsigned char* lds) {
    const int tb = (a.Tp + 63) / 64, db = (a.dh + 63) / 64;
    const int bz = static_cast<int>(i / (tb * db));
    const int rem = static_cast<int>(i % (tb * db));
    qt_tile<STORE, GROUPS>(a, rem % tb, rem / tb, bz, lds);
}

struct ScoreArgs {
    const void* q;        // token t of sequence b at q + b*q_bstride + t*H*d_q
    int64_t q_bstride;
    const void* K1;       // [B][H][n][dh]
    const void* K2;
    const float* knorm;   // [B][H][2][n]
    int B, Tc, n, H, dh, kh;
    float eps;
    int mode;
    uint64_t* cand;       // [B][H][2][Tc][cap]  (e bits << 32 | sub-key)
    int32_t* cnt;         // [B][H][2][Tc]       candidates found (may exceed cap)
    int cap;
    float* qn;            // [B][H][2][Tc]  ||q_half||^2
    float* part;          // [B][H][2][ceil(Tc/tile)][n]
    float* lp;            // [B][H][2][n]   log pbar (row statistic: computed from part, written by
                          //   one workgroup per (sequence, head, half) for the key step)
    int pbar_ntiles;      // row statistic: tiles of the usage partials in part
    QtArgs qt;            // row statistic from stored rows, qt.qT non-NULL: the launch also writes
                          //   the chunk's transposed queries (qt_tiles(qt) workgroups after the
                          //   statistic's)
    int stat_blocks;      // row statistic from stored rows: the statistic's workgroups (set by
                          //   the launcher)
    float* Z;             // [B][H][2][Tc]
    float* m;             // [B][H][2][Tc]
    uint32_t* erow;       // [B][H][2][Tc][n]  e bit patterns (rows mode)
    float* M;             // [B][H][2][Tc]  row maximum of s (dot scoring's softmax)
    int dot;              // dot-product scoring: keys are ord(-s), p = exp(s - M) / Z
    int tile;             // tokens per workgroup (set by launch_score)
};

struct SelectArgs {
    const uint64_t* cand;
    const int32_t* cnt;
    int cap;
    const void* q;        // for the exact recompute of an overflowed list
    int64_t q_bstride;
    const void* K1;
    const void* K2;
    int B, Tc, n, H, dh, kh, k, ncand;
    float eps;
    int32_t* idx;         // [b*iw_bstride + (t*H + h)*k + j]
    float* w;
    int64_t iw_bstride;
    CandTable cand_ab;
    const uint32_t* erow; // non-NULL: whole rows of e ([B][H][2][Tc][n]) instead of candidate lists
    int32_t* usage;       // nullable: usage[b*n*n + slot] += 1 per selected read
    int dot;              // dot-product scoring: keys are ord(-s), pair value -(s1 + s2)
    float* Z;             // whole rows only, nullable: Z_t (and M_t for dot) of every
    float* M;             //   row, computed as k_row_z computes them
};

int score_keep(int kh);   // smallest e kept per lane in the first scoring pass
int score_cap(int kh);    // candidate list capacity per (token, head, half)

struct GatherArgs {
    const void* V;        // [B][N][dv]
    const int32_t* idx;   // [b*iw_bstride + t*H*k + e]
    const float* w;
    int64_t iw_bstride;
    const void* v;        // residual path value: v + b*v_bstride + t*dv
    int64_t v_bstride;
    const float* g;       // g + b*g_bstride + t
    int64_t g_bstride;
    const void* tgt;      // raw target of token t: tgt + b*tgt_bstride + t*dv, t < n_tgt
    int64_t tgt_bstride;
    int n_tgt;            // tokens with a target (per sequence)
    const void* tgt_last; // nullable: target of token Tc-1 at tgt_last + b*tgt_last_bstride
    int64_t tgt_last_bstride;
    float* o;             // o + b*o_bstride + t*dv
    float* vhat;          // nullable, same layout as o
    int64_t o_bstride;
    float* r;             // nullable: residual [B][Tc][dv] when given
    float* vhat2;         // nullable: a second copy of vhat at vhat2 + b*vhat2_bstride + t*dv
    int64_t vhat2_bstride;
    // stream: copies of the token's inputs into the pending chunk (pq nullable)
    const void* q;        // q + (b*q_bstride + t*qrow) elements
    int64_t q_bstride;
    int qrow;             // H*d_q
    void* pq;             // pq + (b*pq_bstride + t*qrow) elements
    int64_t pq_bstride;
    float* pg;            // pg + b*pg_bstride + t
    int64_t pg_bstride;
    void* ptgt;           // v of token t to ptgt + (b*ptgt_bstride + (t + ptgt_shift)*dv), if >= 0
    int64_t ptgt_bstride;
    int ptgt_shift;
    int B, Tc, H, k, dv;
    int64_t N;
    int znorm;
    float znorm_eps;
    int gate_w;           // 1: r = g (vhat - y); 0: r = vhat - y
    int keep_b0;          // k_gather: sequences b >= keep_b0 read value rows with cache-allocating
                          //   loads, earlier ones with streaming (non-temporal) loads
    int held;             // k_gather, bf16 storage: 1 holds a round's rows as their raw bf16
                          //   words (100 rather than 163 registers at d_v = 512), 0 widens them
};

// Capacity of the memory-side last-level cache (MI355X: 256 MB).
constexpr int64_t kLastLevelCacheBytes = int64_t{256} << 20;

// The first sequence of a chunk-gather launch of B sequences whose value rows
// are read into the last-level cache.  The value write that follows reads the
// same rows again; of a launch larger than the cache, only the rows read last
// (its last sequences, up to the cache's capacity) are still there by then,
// so the earlier sequences' rows are streamed past it.
inline int gather_keep_from(int B, int Tc, int H, int k, int dv, int es) {
    const int64_t per_seq = static_cast<int64_t>(Tc) * H * k * dv * es;
    const int64_t fit = per_seq > 0 ? kLastLevelCacheBytes / per_seq : B;
    return static_cast<int>(std::max<int64_t>(0, B - std::max<int64_t>(fit, 1)));
}

struct ResidArgs {        // r = g (vhat - z(tgt)) for t < n_tgt
    const float* vhat;    // vhat + b*vhat_bstride + t*dv
    const float* g;       // g + b*g_bstride + t
    const void* tgt;      // tgt + b*tgt_bstride + t*dv
    float* r;             // [B][Tc][dv]
    int64_t vhat_bstride, g_bstride, tgt_bstride;
    int B, Tc, n_tgt, dv, znorm;
    float znorm_eps;
    int gate_w;
};

struct SortArgs {
    const int32_t* idx;   // first pass source: slot of entry e = idx[b*idx_bstride + e]
    int64_t idx_bstride;
    const uint32_t* kin;  // later passes: keys / values in
    const uint32_t* vin;
    uint32_t* kout;
    uint32_t* vout;
    uint32_t* counts;     // [B][tiles][256]
    int B, M;             // entries per sequence
    int tiles;
    int shift;
    int first;
    uint32_t N;           // slot ids >= N (or < 0) become the sentinel key N
    int items;            // entries per thread: kSortItems or kSortItemsSmall
    int passes;           // 8-bit passes over the keys
    int fuse;             // counts of pass p+1 built by pass p's scatter (integer atomics into
                          //   counts + (p+1)*pass_stride); only pass 0 has a count launch
    int64_t pass_stride;  // entries between the passes' count arrays (fuse)
};

struct ScatterArgs {
    const uint32_t* keys; // sorted slot per position [B][M]
    const uint32_t* vals; // entry id per position [B][M]
    const float* w;       // weights by entry id: w[b*w_bstride + e]
    int64_t w_bstride;
    const float* r;       // residual [B][Tc][dv]
    void* V;              // [B][N][dv]
    int32_t* n_read;      // nullable [B][N]
    float* ph;            // [B][pieces][dv] partial of the run continuing into the piece
    float* pt;            // [B][pieces][dv] partial of the run leaving the piece
    int32_t* pt_start;    // [B][pieces] start position of the leaving run, or -1
    int32_t* ph_end;      // [B][pieces] end position (exclusive) of the entering run, or -1
    int B, M, pieces, H, k, dv, Tc;
    int piece;            // sorted positions per piece (wavefront), <= 64
    uint32_t N;
    float lr, inv_h;
};


struct KgradArgs {
    const void* q;
    int64_t q_bstride;
    const void* qT;       // [B][H][2][dh][Tp] (written in tiles of qt_tile); fp32 storage only
    int Tp;
    void* K1;
    void* K2;
    float* knorm;         // [B][H][2][n], rewritten with the new keys
    const float* qn;      // [B][H][2][Tc]
    const float* Z;
    const float* m;
    const float* lp;      // [B][H][2][n]
    int B, Tc, n, H, dh;
    float eps, lr;
    const float* M;       // [B][H][2][Tc] row maximum of s (dot scoring)
    int dot;
    // Token split: split > 1 runs each 64-key block as `split` workgroups over
    // `per` consecutive 32-token blocks each, which leave their sums in `part`
    // (kgrad_part_floats floats) for k_kgrad_finish to add in split order.
    int split, per;
    float* part;
};

// Token split of the key step for one sequence.  A sequence with fewer than
// kKgradSplitBelow 64-key workgroups (H * 2 * ceil(n/64)) is split by a power
// of two <= kKgradMaxSplit that brings them up to kKgradWgs, with at least
// kKgradMinBlocks 32-token blocks per split.  A wider sequence already gives
// the chip enough workgroups at modest batch sizes, and the partials' round
// trip through memory costs more than the split gains -- unless its chunk is
// long: then each split keeps at least kKgradLongBlocks blocks (a 1024-token
// chunk splits in two; 512 and fewer tokens do not).  The rule reads
// per-sequence sizes only, so a sequence's keys sum in the same order
// whatever the batch around it.  `override` > 0 replaces the power of two
// (still capped by kKgradMaxSplit, which k_kgrad_finish holds in registers,
// and by the block count).  Returns the split and sets *per
// (blocks per split) so that no split is empty.
constexpr int kKgradSplitBelow = 64;
constexpr int kKgradMaxSplit = 8;
constexpr int kKgradWgs = 256;
constexpr int kKgradMinBlocks = 2;
constexpr int kKgradLongBlocks = 16;
inline int kgrad_split(int H, int n, int Tc, int override, int* per) {
    const int nblk = (Tc + 31) / 32;
    const int P = H * 2 * ((n + 63) / 64);
    int s = 1;
    if (override > 0) {
        s = std::min(std::min(override, kKgradMaxSplit), nblk);
    } else if (P < kKgradSplitBelow) {
        while (s < kKgradMaxSplit && P * 2 * s <= kKgradWgs && 2 * s * kKgradMinBlocks <= nblk) s *= 2;
    } else {
        while (s < kKgradMaxSplit && 2 * s * kKgradLongBlocks <= nblk) s *= 2;
    }
    s = std::max(s, 1);
    const int pb = (nblk + s - 1) / s;
    if (per) *per = pb;
    return (nblk + pb - 1) / pb;
}
// Floats of the split partials: per (sequence, head, half, split, key), a
// row of dh gradient sums and one column sum.
inline size_t kgrad_part_floats(int B, int H, int n, int dh, int split) {
    return static_cast<size_t>(B) * H * 2 * split * n * (static_cast<size_t>(dh) + 1);
}

struct KnormArgs {
    const void* K1;
    const void* K2;
    float* knorm;
    int B, H, n, dh;
};

// ---------------------------------------------------------------------------
// launchers (each returns hipGetLastError() after enqueueing)
// ---------------------------------------------------------------------------
hipError_t launch_knorm(const KnormArgs& a, int store, hipStream_t s);
// Tokens per scoring workgroup for B sequences of H heads and Tc tokens on
// the current device: the largest tile whose grid still covers every
// compute unit, else the smallest.
int score_tile(int B, int H, int Tc, bool dot);
// compute units of the current device (cached per device)
int device_cus();
// Statistics of stored rows (rows mode): what = 0 writes Z (and M for dot
// scoring) and the per-64-token usage partials into part; what = 1 writes m
// (needs lp), with the transposed queries of a.qt when a.qt.qT is set.
hipError_t launch_row_stats(const ScoreArgs& a, int what, int store, hipStream_t s);
// Gradient of the retrieval output w.r.t. q, v and g for T tokens of B
// sequences; per-sequence strides in elements:
//   q, dq (f32):         + b*q_bstride + (t*H + h)*2*dh
//   v, dO, dv_out (f32): + b*v_bstride + t*dv
//   g, dg:               + b*g_bstride + t
//   idx, w:              + b*iw_bstride + (t*H + h)*k
struct BackwardArgs {
    const void* q;
    int64_t q_bstride;
    const void* v;
    int64_t v_bstride;
    const float* g;
    int64_t g_bstride;
    const int32_t* idx;
    const float* w;
    int64_t iw_bstride;
    const void* K1;
    const void* K2;
    const void* V;
    const float* dO;
    float* dq;
    float* dv_out;
    float* dg;
    int B, T, n, H, dh, dv, k;
    int64_t N;
    float eps;
    int dot;
};
hipError_t launch_backward(const BackwardArgs& a, int store, hipStream_t s);

hipError_t launch_score(const ScoreArgs& a, int store, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int store, hipStream_t s);
// Whole-row selection and the value read of the same few tokens fused in one
// workgroup per token (decode), for 2*H and the read's parts within kSgWaves
// wavefronts (select_gather_fits); the same results as launch_select
// followed by launch_gather.
constexpr int kSgWaves = 16;
bool select_gather_fits(int H, int k);
hipError_t launch_select_gather(const SelectArgs& a, const GatherArgs& ga, int store, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, int store, hipStream_t s);
hipError_t launch_resid(const ResidArgs& a, int store, hipStream_t s);
hipError_t launch_sort_pass(const SortArgs& a, hipStream_t s);
hipError_t launch_scatter(const ScatterArgs& a, int store, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int64_t count, int32_t value, hipStream_t s);
// metrics[b] = {coverage, collision, KLD, accesses} of usage[b][0..N); reset clears usage;
// scratch holds B*kUsageParts partial sums of 32 bytes
constexpr int kUsageParts = 64;
hipError_t launch_usage_metrics(int32_t* usage, int B, int64_t N, void* scratch, double* metrics, int reset,
                                hipStream_t s);
// height rows of width_bytes (a multiple of 4) from src + y*spitch to dst + y*dpitch
hipError_t launch_copy2d(void* dst, int64_t dpitch, const void* src, int64_t spitch, int64_t width_bytes,
                         int64_t height, hipStream_t s);
hipError_t launch_kgrad(const KgradArgs& a, int store, hipStream_t s);
// the transposed query halves alone (tiles of qt_tile)
hipError_t launch_qt(const QtArgs& a, int store, hipStream_t s);

constexpr int kSortItems = 8;                  // entries per thread
constexpr int kSortTile = 256 * kSortItems;    // entries per sort workgroup
// Sorts whose 2048-entry tiles give fewer than kSortMinTiles workgroups
// (a single long sequence, a small batch) use 512-entry tiles instead.
constexpr int kSortItemsSmall = 2;
constexpr int kSortTileSmall = 256 * kSortItemsSmall;
constexpr int kSortMinTiles = 128;
constexpr int kSortFuseTiles = 64;             // at most B*tiles for next-pass counts by the scatters
inline int sort_items(int B, int M) {
    return static_cast<long long>(B) * ((M + kSortTile - 1) / kSortTile) < kSortMinTiles ? kSortItemsSmall
                                                                                          : kSortItems;
}
constexpr int kPiece = 64;                     // sorted positions per scatter wavefront (at most)
// Positions per scatter piece for a sequence of M sorted reads: 64, or 32 /
// 16 when 64-position pieces would give a sequence fewer than kPieceWaves
// wavefronts.  It depends on M only, so a sequence's write sums in the same
// order whatever the batch around it.
constexpr int kPieceWaves = 1024;
inline int scatter_piece(int M) {
    int piece = kPiece;
    while (piece > 16 && (M + piece - 1) / piece < kPieceWaves) piece >>= 1;
    return piece;
}

}  // namespace fwpkm
