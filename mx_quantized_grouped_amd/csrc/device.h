// Device helpers shared by the MX MoE kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// K elements consumed by one block-scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
constexpr int KSTEP = 128;
// Operand formats of a grouped GEMM: the weight (B) element, and for the MX formats the
// activation (A) element: MXFP8 weights and activations, MXFP4 weights with MXFP8 activations,
// bf16 both, and MXFP4 weights with MXFP4 activations (W4A4).
enum WFmt { WF_FP8 = 0, WF_FP4 = 1, WF_BF16 = 2, WF_FP4A4 = 3 };
__host__ __device__ constexpr bool w_is_fp4(int wf) { return wf == WF_FP4 || wf == WF_FP4A4; }
__host__ __device__ constexpr bool a_is_fp4(int wf) { return wf == WF_FP4A4; }

// ---------------------------------------------------------------------------- direct LDS loads
// Raw buffer descriptor words (the raw-buffer format word of gfx9: loads past num_bytes return
// zero) for the asm loads below.
__device__ __forceinline__ v4i rsrc_words(const void* base, uint32_t num_bytes) {
  const uint64_t a = (uint64_t)base;
  return v4i{(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xFFFFu), (int)num_bytes, 0x00020000};
}

// Direct global -> LDS loads: lane i's 16 (or 4) bytes land at LDS byte lds + 16 i (or 4 i).
// They are issued from asm so that the compiler does not add its own (all-outstanding) waits
// before every LDS read; the caller tracks completion with explicit s_waitcnt vmcnt.
__device__ __forceinline__ void lds_load16(v4i rsrc, uint32_t lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "m0");
}
__device__ __forceinline__ void lds_load4(v4i rsrc, uint32_t lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               ::"s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "m0");
}

// ---------------------------------------------------------------------------- lane helpers
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0));
}

// ---------------------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two fp32 values to bf16, round to nearest even, a in the low half: one v_cvt_pk_bf16_f32 on
// gfx950 (the integer form above takes about four instructions per value plus the packing).
typedef float v2f_t __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f_t{a, b}, v2bf_t));
}

// ---------------------------------------------------------------------------- MX encoding
// floor(log2(a)) for finite a > 0 (fp32 subnormals included), from the exponent bits.
__device__ __forceinline__ int floor_log2(float a) {
  uint32_t u = __float_as_uint(a);
  int e = (int)((u >> 23) & 0xFF);
  if (e == 0) return 31 - __clz(u & 0x7FFFFF) - 149;
  return e - 127;
}

// Shared exponent of an MX block: floor(log2(amax)) - emax_elem, clamped to [-127, 127];
// an all-zero block gets -127 (scale byte 0). amax is a block maximum of magnitudes (>= 0,
// finite). Branch-free: zero takes the subnormal formula, 31 - clz(0) - 149 = -150, which the
// clamp turns into -127.
template <int EMAX>
__device__ __forceinline__ int mx_shared_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int e = (int)(u >> 23);
  const int lg = e ? e - 127 : 31 - (int)__clz(u & 0x7FFFFFu) - 149;
  const int se = lg - EMAX;
  return se < -127 ? -127 : (se > 127 ? 127 : se);
}

// E2M1 magnitude code of a in [0, 6].
__device__ __forceinline__ uint32_t e2m1_mag(float a) {
  if (a < 1.0f) return (uint32_t)__builtin_rintf(a * 2.0f);          // 0, 0.5, 1.0 (code 2)
  uint32_t u = __float_as_uint(a);
  u += 0x1FFFFFu + ((u >> 22) & 1u);                                 // keep 1 mantissa bit
  return (((u >> 23) - 126u) << 1) | ((u >> 22) & 1u);               // rebias 127 -> 1
}
// E4M3 codes of two elements of a block with shared exponent se, element a in the low byte: the
// nearest code of x / 2^se, ties to even, saturating at 448, sign kept. x / 2^se is exact (a
// power-of-two scaling of a finite value) and clamped to +-448, then the hardware's packed E4M3
// conversion rounds it to nearest even. The device quantisers' codes are checked bit-exactly
// against the reference rule on every finite bf16 value and on fp32 blocks with exact ties.
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b, int se) {
  const float ca = fminf(fmaxf(ldexpf(a, -se), -448.0f), 448.0f);
  const float cb = fminf(fmaxf(ldexpf(b, -se), -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false) & 0xFFFFu;
}
// Four codes packed little-endian into a dword.
__device__ __forceinline__ uint32_t e4m3_quad(float a, float b, float c, float d, int se) {
  const float ca = fminf(fmaxf(ldexpf(a, -se), -448.0f), 448.0f);
  const float cb = fminf(fmaxf(ldexpf(b, -se), -448.0f), 448.0f);
  const float cc = fminf(fmaxf(ldexpf(c, -se), -448.0f), 448.0f);
  const float cd = fminf(fmaxf(ldexpf(d, -se), -448.0f), 448.0f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, lo, true);
}
// E2M1 element code of x in a block with shared exponent se (sign kept, saturating at 6).
__device__ __forceinline__ uint32_t e2m1_code(float x, int se) {
  float v = ldexpf(x, -se);
  uint32_t m = e2m1_mag(fminf(fabsf(v), 6.0f));
  return m | ((__float_as_uint(v) >> 28) & 0x8u);
}

// E2M1 codes of columns n and 16 + n of a 32-column MX block whose 16 columns pairs are spread over
// the 16 lanes of a DPP row (lane n holds columns n and 16 + n), packed two codes per byte,
// element 2i in the low nibble: an even lane n returns byte n / 2 (columns n, n + 1) in bits 0-7
// and byte 8 + n / 2 (columns 16 + n, 17 + n) in bits 8-15. All 64 lanes must take part.
__device__ __forceinline__ uint32_t e2m1_pack_pair(float a0, float a1, int se) {
  const uint32_t q = e2m1_code(a0, se) | (e2m1_code(a1, se) << 8);
  // quad_perm [1,0,3,2]: the codes of the neighbouring column pair
  const uint32_t nb = (uint32_t)__builtin_amdgcn_update_dpp((int)q, (int)q, 0xB1, 0xF, 0xF, false);
  return (q & 0x0F0Fu) | ((nb & 0x0F0Fu) << 4);
}

// ---------------------------------------------------------------------------- layouts
// Scales of an activation / intermediate row are stored in K-block order, one byte per 32 elements,
// in rows padded to a multiple of 16 bytes: the four K-blocks of one 128-K MFMA step are one dword.
__device__ __host__ __forceinline__ int round_up(int a, int b) { return (a + b - 1) / b * b; }

}  // namespace mxmoe
