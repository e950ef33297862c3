// bf16 packing and the RoPE3D pair rotation used by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vdit_internal.hpp"

namespace vdit {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950 converts pairs in hardware).
__device__ inline uint32_t pack_bf16x2(float a, float b) {
    f32x2 f = {a, b};
    bf16x2 h = __builtin_convertvector(f, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ inline u32x4 pack_bf16x8(const float x[8]) {
    u32x4 u;
    u[0] = pack_bf16x2(x[0], x[1]);
    u[1] = pack_bf16x2(x[2], x[3]);
    u[2] = pack_bf16x2(x[4], x[5]);
    u[3] = pack_bf16x2(x[6], x[7]);
    return u;
}

__device__ inline void unpack_bf16x8(u32x4 u, float x[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, u[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xFFFF0000u);
    }
}

// Rotates the 4 channel pairs pair0 .. pair0+3 held in x[8] (pair e = x[2e], x[2e+1]) of a
// token at global position (t, h, w).  Channel groups are [t | h | w]; pair j of a group
// of width d turns by p * theta^(-2j/d), read from the precomputed (cos, sin) tables
// ("Accelerating Video Generation Inference ...", section 2.C, precomputed RoPE;
// "Timeripple ...", Metodologia 1, channel groups per axis).
__device__ inline void rope_rotate8(const RopeDev& r, int32_t pair0, int32_t t, int32_t h, int32_t w, float x[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        int32_t p = pair0 + e;
        float2 cs;
        if (p < r.pairs_t) {
            cs = r.tab_t[(int64_t)t * r.pairs_t + p];
        } else if (p < r.pairs_t + r.pairs_h) {
            cs = r.tab_h[h * r.pairs_h + (p - r.pairs_t)];
        } else {
            cs = r.tab_w[w * r.pairs_w + (p - r.pairs_t - r.pairs_h)];
        }
        float x0 = x[2 * e], x1 = x[2 * e + 1];
        x[2 * e] = x0 * cs.x - x1 * cs.y;
        x[2 * e + 1] = x0 * cs.y + x1 * cs.x;
    }
}

}  // namespace vdit
