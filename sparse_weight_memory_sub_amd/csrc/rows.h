// rows.h -- loads and stores of d_v-rows spread over a wavefront: lane l
// owns elements [l*EPL, (l+1)*EPL) of the row, so one row is one coalesced
// access of the wavefront.  Storage is fp32 or bf16 (widened exactly).
#pragma once

#include "fwpkm_internal.h"

namespace fwpkm {

template <int STORE, int EPL, bool NT = false>
__device__ __forceinline__ void ldrow(const void* base, size_t off, float (&x)[EPL]) {
    if constexpr (STORE == kF32) {
        const float* p = static_cast<const float*>(base) + off;
        if constexpr (EPL % 4 == 0) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4) {
                const uint4 v = ld16<NT>(p + i);
                x[i] = __uint_as_float(v.x); x[i + 1] = __uint_as_float(v.y);
                x[i + 2] = __uint_as_float(v.z); x[i + 3] = __uint_as_float(v.w);
            }
        } else if constexpr (EPL == 2) {
            const float2 v = *reinterpret_cast<const float2*>(p);
            x[0] = v.x; x[1] = v.y;
        } else {
            x[0] = p[0];
        }
    } else {
        const uint16_t* p = static_cast<const uint16_t*>(base) + off;
        if constexpr (EPL == 8) {
            const uint4 v = ld16<NT>(p);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = __uint_as_float(w[i] << 16);
                x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        } else if constexpr (EPL == 4) {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xffff0000u);
            x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xffff0000u);
        } else if constexpr (EPL == 2) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
            x[0] = __uint_as_float(v << 16); x[1] = __uint_as_float(v & 0xffff0000u);
        } else {
            x[0] = bf16_to_f32(p[0]);
        }
    }
}

template <int EPL>
__device__ __forceinline__ void stf(float* p, const float (&x)[EPL]) {
    if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < EPL; i += 4)
            *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
    } else if constexpr (EPL == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    } else {
        p[0] = x[0];
    }
}

}  // namespace fwpkm
