// MX-FP8: OCP E4M3 codes with one power-of-two scale per 32 values (E8M0 byte, bias 127).
// Device helpers shared by the quantisation kernel and the FP8 grouped GEMM's epilogue, so
// a bit-exact check of the former covers the latter's conversion too.
#pragma once

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ uint32_t mag_bits(float v) {
  return __float_as_uint(v) & 0x7fffffffu;
}

// Shared exponent X of a block whose largest magnitude has the bit pattern `amax` (sign
// cleared; integer order of such patterns is the order of the values): floor(log2(amax))
// - 8, -127 for amax = 0, clamped to [-127, 127]. The scale byte is X + 127.
__device__ __forceinline__ int mx_exponent(uint32_t amax) {
  const int fl_norm = (int)(amax >> 23) - 127;
  const int fl_sub = (31 - (int)__builtin_clz(amax | 1u)) - 149;   // m * 2^-149
  const int fl = amax >= 0x00800000u ? fl_norm : fl_sub;
  const int x = fl - 8;
  return amax == 0 ? -127 : (x < -127 ? -127 : (x > 127 ? 127 : x));
}

// Codes of four values of one block: v / 2^x (exact: a power-of-two scaling of a value at
// most 2^9 in magnitude), clamped to +-448, converted by the hardware's fp32 -> E4M3
// instruction (round to nearest, ties to even). Clamping first gives the saturating
// conversion: every magnitude of 448 or more has 448 as its saturated nearest value.
// The sign bit is v's, also for values that round to zero.
__device__ __forceinline__ uint32_t mx_pack4(float v0, float v1, float v2, float v3, int x) {
  auto sc = [x](float v) __attribute__((always_inline)) {
    return __builtin_amdgcn_fmed3f(__builtin_amdgcn_ldexpf(v, -x), -448.f, 448.f);
  };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sc(v0), sc(v1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sc(v2), sc(v3), w, true);
  return (uint32_t)w;
}

}  // namespace moe
