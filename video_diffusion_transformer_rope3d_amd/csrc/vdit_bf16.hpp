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
// (cos, sin) of channel pair p at position (t, h, w): the pair's axis table, row = the
// position on that axis.  Branch-free (selects), so that the loads of several pairs can be
// issued together.  The tables' addresses and row lengths are first read into scalar
// registers (every kernel passes one RopeDev to all its lanes): left as a choice between
// fields of the struct, the compiler loads the chosen field per lane, one dependent global
// load ahead of every table read.
typedef __attribute__((address_space(1))) const float rope_gfloat;  // global memory
__device__ inline rope_gfloat* rope_uniform_ptr(const float2* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<rope_gfloat*>(((uint64_t)hi << 32) | lo);
}

__device__ inline float2 rope_cs(const RopeDev& r, int32_t p, int32_t t, int32_t h, int32_t w) {
    const int32_t nt = __builtin_amdgcn_readfirstlane(r.pairs_t), nh = __builtin_amdgcn_readfirstlane(r.pairs_h);
    const int32_t nw = __builtin_amdgcn_readfirstlane(r.pairs_w);
    rope_gfloat* tt = rope_uniform_ptr(r.tab_t);
    rope_gfloat* th = rope_uniform_ptr(r.tab_h);
    rope_gfloat* tw = rope_uniform_ptr(r.tab_w);
    const bool in_t = p < nt, in_h = p < nt + nh;
    rope_gfloat* tab = in_t ? tt : (in_h ? th : tw);
    const int32_t coord = in_t ? t : (in_h ? h : w);
    const int32_t pitch = in_t ? nt : (in_h ? nh : nw);
    const int32_t col = in_t ? p : (in_h ? p - nt : p - nt - nh);
    rope_gfloat* e = tab + 2 * ((int64_t)coord * pitch + col);
    return make_float2(e[0], e[1]);
}

__device__ inline void rope_apply(float2 cs, float& x0, float& x1) {
    const float a = x0, b = x1;
    x0 = a * cs.x - b * cs.y;
    x1 = a * cs.y + b * cs.x;
}

__device__ inline void rope_rotate8(const RopeDev& r, int32_t pair0, int32_t t, int32_t h, int32_t w, float x[8]) {
    float2 cs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) cs[e] = rope_cs(r, pair0 + e, t, h, w);
#pragma unroll
    for (int e = 0; e < 4; ++e) rope_apply(cs[e], x[2 * e], x[2 * e + 1]);
}

}  // namespace vdit
