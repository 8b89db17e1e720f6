// Device side of MX quantisation (see quant.hip for the rule). Weight blocks: one thread per block
// of 32 consecutive values; activation blocks: four lanes per block.
#pragma once
#include "device.h"

namespace mxmoe {

// Load 32 consecutive source elements as fp32.
template <bool F32>
__device__ __forceinline__ void load32(const void* src, size_t off, float* v) {
  if (F32) {
    const v4f* p = (const v4f*)((const float*)src + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v4f q = p[i];
      v[4 * i] = q[0]; v[4 * i + 1] = q[1]; v[4 * i + 2] = q[2]; v[4 * i + 3] = q[3];
    }
  } else {
    const v4i* p = (const v4i*)((const uint16_t*)src + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v4i q = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t u = (uint32_t)q[j];
        v[8 * i + 2 * j] = __uint_as_float(u << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(u & 0xFFFF0000u);
      }
    }
  }
}

__device__ __forceinline__ float amax32(const float* v) {
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
  return a;
}

// 32 E4M3 codes packed little-endian into 8 dwords.
__device__ __forceinline__ void encode_fp8_32(const float* v, int se, uint32_t* out) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    out[i] = e4m3_quad(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], se);
}
// 32 E2M1 codes, element 2i in the low nibble of byte i, packed into 4 dwords.
__device__ __forceinline__ void encode_fp4_32(const float* v, int se, uint32_t* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t d = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) d |= e2m1_code(v[8 * i + j], se) << (4 * j);
    out[i] = d;
  }
}

// Activation block (t, kb) of bf16 x [T, H] -> E4M3 codes in xq [T, H] (A4: E2M1 codes, two per
// byte, in xq [T, H / 2]) and the scale byte in xs [T, srs] (K-block order); optionally clears the
// matching 32 floats of zero_out [T, H]. Four consecutive lanes (a DPP quad) share a block, lane
// part p holding elements 8p .. 8p + 7, so each load instruction of a wave reads 1 KiB of
// consecutive bytes and each store writes consecutive bytes (one thread per block read 16-byte
// pieces 64 bytes apart: the 8K-token quantisation ran at ~3 TB/s). The block maximum is exact
// whatever the order, so the codes are those of the one-thread-per-block rule.
__device__ __forceinline__ void quant_act_part(const uint16_t* x, size_t t, int kb, int part,
                                               int H, uint8_t* xq, uint8_t* xs, int srs, bool a4,
                                               float* zero_out) {
  const size_t off = t * H + (size_t)kb * 32 + 8 * part;
  if (xq) {
    const v4i q = *(const v4i*)(x + off);
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t u = (uint32_t)q[j];
      v[2 * j] = __uint_as_float(u << 16);
      v[2 * j + 1] = __uint_as_float(u & 0xFFFF0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    // quad_perm [1,0,3,2], then [2,3,0,1]: the maximum over the block's four lanes (non-negative
    // floats order like their bit patterns; every source lane is inside the quad)
    uint32_t mu = __float_as_uint(m);
    mu = max(mu, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mu, 0xB1, 0xF, 0xF, true));
    mu = max(mu, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mu, 0x4E, 0xF, 0xF, true));
    m = __uint_as_float(mu);
    if (a4) {
      const int se = mx_shared_exp<2>(m);
      if (part == 0) xs[t * srs + kb] = (uint8_t)(se + 127);
      uint32_t d = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) d |= e2m1_code(v[j], se) << (4 * j);
      *(uint32_t*)(xq + off / 2) = d;
    } else {
      const int se = mx_shared_exp<8>(m);
      if (part == 0) xs[t * srs + kb] = (uint8_t)(se + 127);
      *(uint2*)(xq + off) = uint2{e4m3_quad(v[0], v[1], v[2], v[3], se),
                                  e4m3_quad(v[4], v[5], v[6], v[7], se)};
    }
  }
  if (zero_out) {
    v4f* z = (v4f*)(zero_out + off);
    z[0] = v4f{0.f, 0.f, 0.f, 0.f};
    z[1] = v4f{0.f, 0.f, 0.f, 0.f};
  }
}

}  // namespace mxmoe
