// mfma_frag.h -- 16x16 MFMA tiles over 32-wide k-blocks for bf16 and fp32
// operands on gfx950.
//
// Lane l of a wavefront owns row/column (l % 16) of a 16-wide operand tile
// and k-group g = l / 16.  A k-block is 32 wide; each lane holds 8 of its
// k-elements.  For an operand row of d elements (d/32 k-blocks) the blocks
// are taken in pairs: lane group g reads the 16 consecutive elements
// [64*s2 + 16*g, +16) of its row with one 32-byte (bf16) load, the first 8
// for block 2*s2 and the last 8 for block 2*s2 + 1, so the four groups of a
// row cover a whole 128-byte line.  (A single block, d = 32, uses
// [8*g, +8).)  A and B use the same map, so the products pair up whatever
// order the instruction sums them in.  The 16x16 fp32 result is spread as
// acc[i] = C[row 4*(l/16) + i][column l % 16].
#pragma once

#include "fwpkm_internal.h"

namespace fwpkm {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short v4i16_t;

template <int STORE> struct Frag;
template <> struct Frag<kBF16> {
    u32x4_t v;  // 8 bf16, element j in bits 16*(j%2) of word j/2
};
template <> struct Frag<kF32> {
    float v[8];
};

template <int STORE> __device__ __forceinline__ void frag_zero(Frag<STORE>& f);
template <> __device__ __forceinline__ void frag_zero<kBF16>(Frag<kBF16>& f) {
    f.v = u32x4_t{0u, 0u, 0u, 0u};
}
template <> __device__ __forceinline__ void frag_zero<kF32>(Frag<kF32>& f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = 0.f;
}

// 8 consecutive storage elements starting at p (16-byte aligned for bf16,
// 32-byte aligned for fp32).
template <int STORE> __device__ __forceinline__ void frag_load(Frag<STORE>& f, const void* p);
template <> __device__ __forceinline__ void frag_load<kBF16>(Frag<kBF16>& f, const void* p) {
    f.v = *reinterpret_cast<const u32x4_t*>(p);
}
template <> __device__ __forceinline__ void frag_load<kF32>(Frag<kF32>& f, const void* p) {
    const float4* s = reinterpret_cast<const float4*>(p);
    float4 a = s[0], b = s[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// All DHS fragments of one operand row (d = 32*DHS storage elements starting
// at `row`, 16-byte aligned) for lane group g, in the k-block map above.
template <int STORE, int DHS>
__device__ __forceinline__ void load_row_frags(Frag<STORE> (&f)[DHS], const unsigned char* row, int g) {
    constexpr int ES = Store<STORE>::kBytes;
    if constexpr (DHS == 1) {
        frag_load<STORE>(f[0], row + 8 * g * ES);
    } else {
#pragma unroll
        for (int s2 = 0; s2 < DHS / 2; ++s2) {
            const unsigned char* p = row + (64 * s2 + 16 * g) * ES;
            frag_load<STORE>(f[2 * s2], p);
            frag_load<STORE>(f[2 * s2 + 1], p + 8 * ES);
        }
    }
}

// Sum of squares of the fragment's elements (fp32).
template <int STORE> __device__ __forceinline__ float frag_sumsq(const Frag<STORE>& f);
template <> __device__ __forceinline__ float frag_sumsq<kBF16>(const Frag<kBF16>& f) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float lo = __uint_as_float(f.v[j] << 16), hi = __uint_as_float(f.v[j] & 0xffff0000u);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
    }
    return s;
}
template <> __device__ __forceinline__ float frag_sumsq<kF32>(const Frag<kF32>& f) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s = fmaf(f.v[j], f.v[j], s);
    return s;
}

// acc += A * B over one 32-wide k-block.
__device__ __forceinline__ void mma(const Frag<kBF16>& a, const Frag<kBF16>& b, f32x4_t& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.v),
                                                   __builtin_bit_cast(bf16x8_t, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(const Frag<kF32>& a, const Frag<kF32>& b, f32x4_t& acc) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Swizzled LDS images of operand tiles, filled by direct global-to-LDS loads
// ---------------------------------------------------------------------------
//
// A tile of ROWS rows of CPR 16-byte chunks is stored row after row, with
// the chunk index of row R permuted by an xor, chunk c at R*CPR + (c ^ swz(R)).
// The sixteen lanes r = 0..15 of a lane group read the same chunk of sixteen
// consecutive rows.  The swizzle puts those reads in sixteen distinct
// 16-byte bank groups of 256 bytes, and each half (lanes r = 0..7, 8..15) in
// eight distinct groups of 128 bytes, so a 16-byte read meets no bank
// conflict whether the LDS serves it sixteen or eight lanes at a time:
//   CPR >= 16: swz(R) = R & 15;
//   CPR = 8:   swz(R) = ((R >> 1) ^ (R << 2)) & 7;
//   CPR = 4:   swz(R) = ((R >> 2) ^ (R >> 1)) & 3.
// (Measured on the key step's 4-chunk transposed tile: (R >> 2) & 3, which
// is conflict-free only sixteen lanes at a time, left the LDS with bank
// conflicts in most of its busy cycles.)

template <int CPR, bool NARROW = false>
__device__ __forceinline__ int swz(int R) {
    static_assert(CPR == 4 || CPR == 8 || CPR >= 16, "rows of 4, 8 or at least 16 chunks");
    if constexpr (CPR >= 16) return R & 15;
    else if constexpr (CPR == 8) return ((R >> 1) ^ (R << 2)) & 7;
    else return ((R >> 2) ^ (R >> 1)) & 3;
}

// Copies rows [0, ROWS) of a strided source (row R at src + R*stride bytes;
// rows R >= nvalid are skipped and keep whatever the image held) into the
// image at dst.  Each wavefront instruction fills 64 consecutive chunk
// positions, lane L position 64*j + L, from the global chunk that belongs
// there; the NW wavefronts of the workgroup take instructions in turn.
template <int CPR, int ROWS, int NW, bool NARROW>
__device__ __forceinline__ void dma_rows(unsigned char* dst, const unsigned char* src, uint32_t stride, int nvalid,
                                         int wave, int lane) {
    constexpr int NINST = ROWS * CPR / 64;
    static_assert(NINST >= 1 && (ROWS * CPR) % 64 == 0, "tile must be a whole number of 1 KiB pieces");
    const bool full = nvalid >= ROWS;  // the usual case: no per-lane row check
#pragma unroll
    for (int j = 0; j < NINST; j += NW) {
        const int jj = j + wave;
        if (NINST % NW == 0 || jj < NINST) {
            const int p = 64 * jj + lane;
            const int R = p / CPR, cs = p % CPR;
            const int c = cs ^ swz<CPR>(R);
            const void* g = reinterpret_cast<const void*>(
                src + (static_cast<uint32_t>(R) * stride + static_cast<uint32_t>(c) * 16u));
            if (full) {
                __builtin_amdgcn_global_load_lds(g, dst + 64 * jj * 16, 16, 0, 0);
            } else if (R < nvalid) {
                __builtin_amdgcn_global_load_lds(g, dst + 64 * jj * 16, 16, 0, 0);
            }
        }
    }
}

// Per-lane byte offsets of the k-block fragments of row r (0..15) of an
// image of 32*DHS-element rows, for lane group g.  Fragment s = 2*sp + (s & 1)
// (k-block pair sp) of row tile ct (rows 16*ct .. +15) starts at
//   bf16: base[2*(s & 1) + (sp & 1)] + imm(ct, s)
//   fp32: its two 16-byte halves at base[2*(s & 1) + j] + imm(ct, s), j = 0, 1.
// For bf16 rows of 16 or more chunks the xor also flips bit 3 of the chunk
// index (the low bit of sp) in rows 8..15; that is +8 or -8 chunks depending
// on the parity of sp, so it is folded into the two bases of each parity.
template <int STORE, int DHS>
struct FragBase {
    static constexpr int CPR = 32 * DHS * Store<STORE>::kBytes / 16;
    uint32_t base[4];
    __device__ __forceinline__ FragBase(int r, int g) {
        const int f = swz<CPR>(r);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            int pos;
            if constexpr (STORE == kBF16) {
                const int s1 = q >> 1, spp = q & 1;
                if constexpr (DHS == 1) {
                    pos = r * CPR + (g ^ f);
                } else if constexpr (CPR < 16) {
                    pos = r * CPR + ((2 * g + s1) ^ f);
                } else {
                    const int hb = (r >> 3) & 1;
                    pos = r * CPR + ((2 * g + s1) ^ (r & 7)) + 8 * ((spp ^ hb) - spp);
                }
            } else {
                const int s1 = q >> 1, j = q & 1;
                if constexpr (DHS == 1) pos = r * CPR + ((2 * g + j) ^ f);
                else pos = r * CPR + ((4 * g + 2 * s1 + j) ^ f);
            }
            base[q] = static_cast<uint32_t>(pos) * 16u;
        }
    }
    static __device__ __forceinline__ constexpr uint32_t imm(int ct, int s) {
        if constexpr (STORE == kBF16)
            return static_cast<uint32_t>(ct * 16 * CPR + (DHS == 1 ? 0 : 8 * (s >> 1))) * 16u;
        else
            return static_cast<uint32_t>(ct * 16 * CPR + (DHS == 1 ? 0 : 16 * (s >> 1))) * 16u;
    }
};

// Fragment s of row tile ct from the image at img.
template <int STORE, int DHS>
__device__ __forceinline__ void lds_frag(Frag<STORE>& f, const unsigned char* img, const FragBase<STORE, DHS>& fb,
                                         int ct, int s) {
    const uint32_t im = FragBase<STORE, DHS>::imm(ct, s);
    if constexpr (STORE == kBF16) {
        const int q = (DHS == 1) ? 0 : 2 * (s & 1) + ((s >> 1) & 1);
        f.v = *reinterpret_cast<const u32x4_t*>(img + fb.base[q] + im);
    } else {
        const int q = (DHS == 1) ? 0 : 2 * (s & 1);
        const float4 x = *reinterpret_cast<const float4*>(img + fb.base[q] + im);
        const float4 y = *reinterpret_cast<const float4*>(img + fb.base[q + 1] + im);
        f.v[0] = x.x; f.v[1] = x.y; f.v[2] = x.z; f.v[3] = x.w;
        f.v[4] = y.x; f.v[5] = y.y; f.v[6] = y.z; f.v[7] = y.w;
    }
}

// f <- -2 f, exactly (a power-of-two scaling of representable values).
__device__ __forceinline__ void frag_scale_m2(Frag<kBF16>& f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float lo = -2.f * __uint_as_float(f.v[j] << 16);
        const float hi = -2.f * __uint_as_float(f.v[j] & 0xffff0000u);
        f.v[j] = pack_bf16x2(lo, hi);
    }
}
__device__ __forceinline__ void frag_scale_m2(Frag<kF32>& f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] *= -2.f;
}

}  // namespace fwpkm
