// Device-side building blocks shared by the gfx950 kernels: bf16 vector
// types, the 32x32x16 bf16 MFMA, 16-byte global loads, and the key order
// used when a tile is stored transposed in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sigattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum Variant { kSigmoid = 0, kSoftmax = 1, kSoftmax1 = 2 };
enum Bias { kBiasNone = 0, kBiasLogSeqlen = 1, kBiasLogPadlen = 2 };

// D[32x32] += A[32x16] * B[16x32], bf16 inputs, fp32 accumulation.
// Lane l holds A[l % 32][8 * (l / 32) + e] and B[8 * (l / 32) + e][l % 32]
// for e = 0..7; acc[4 * i + j] is D[8 * i + 4 * (l / 32) + j][l % 32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int clamp_len(int n, int L) { return n < 0 ? 0 : (n > L ? L : n); }

// Position of key x (0..15 inside a group of 16) in a transposed LDS row.
// The C fragment of a 32x32 MFMA gives lane half h the rows 4h..4h+3 and
// 8+4h..8+4h+3 of each 16-row group; storing the keys with bits 2 and 3
// swapped makes those 8 keys one contiguous 16-byte run, so the transposed
// operand of the next MFMA is a single 128-bit LDS read.
__device__ __forceinline__ int perm16(int x) {
    return (x & ~15) | (x & 3) | ((x & 4) << 1) | ((x & 8) >> 1);
}

__device__ __forceinline__ uint4 load16(const bf16 *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

__device__ __forceinline__ bf16x8 pack8(const float *x) {
    f32x2 a = {x[0], x[1]}, b = {x[2], x[3]}, c = {x[4], x[5]}, d = {x[6], x[7]};
    bf16x2 pa = __builtin_convertvector(a, bf16x2);
    bf16x2 pb = __builtin_convertvector(b, bf16x2);
    bf16x2 pc = __builtin_convertvector(c, bf16x2);
    bf16x2 pd = __builtin_convertvector(d, bf16x2);
    bf16x8 r = {pa[0], pa[1], pb[0], pb[1], pc[0], pc[1], pd[0], pd[1]};
    return r;
}

__device__ __forceinline__ bf16x4 pack4(float x0, float x1, float x2, float x3) {
    f32x2 a = {x0, x1}, b = {x2, x3};
    bf16x2 pa = __builtin_convertvector(a, bf16x2);
    bf16x2 pb = __builtin_convertvector(b, bf16x2);
    bf16x4 r = {pa[0], pa[1], pb[0], pb[1]};
    return r;
}

// sigma(s) with s = acc * scale + beta, evaluated as 1 / (1 + 2^u) where
// u = acc * c1 + c0, c1 = -scale * log2(e), c0 = -beta * log2(e).
__device__ __forceinline__ float sigmoid_from(float acc, float c1, float c0) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(fmaf(acc, c1, c0)));
}

__device__ __forceinline__ float bias_value(int mode, int n, int L) {
    if (mode == kBiasLogSeqlen) return -logf((float)n);
    if (mode == kBiasLogPadlen) return -logf((float)L);
    return 0.0f;
}

}  // namespace sigattn
