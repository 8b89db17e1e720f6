// Final rounding of the combined output to bf16. With per-slot rows (fp32 or bf16) the k+1 slot
// contributions of a token are summed here in fp32 in slot order (a fixed order, so the result is
// reproducible); with the atomic combine the token-major fp32 accumulator is only converted.
#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

// One thread per 8 consecutive output columns.
template <int COMBINE>
__global__ __launch_bounds__(256) void k_finalize(const void* out, int T, int H, int k1,
                                                  uint16_t* y) {
  const int per_row = H / 8;
  size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * per_row) return;
  size_t t = idx / per_row;
  int c = (int)(idx - t * per_row) * 8;
  float s[8];
  if (COMBINE == 1) {
    const float* out32 = (const float*)out;
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.f;
    for (int j = 0; j < k1; ++j) {
      const v4f* p = (const v4f*)(out32 + (t * k1 + j) * H + c);
      v4f a = p[0], b = p[1];
      s[0] += a[0]; s[1] += a[1]; s[2] += a[2]; s[3] += a[3];
      s[4] += b[0]; s[5] += b[1]; s[6] += b[2]; s[7] += b[3];
    }
  } else if (COMBINE == 3) {
    const uint16_t* out16 = (const uint16_t*)out;
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.f;
    for (int j = 0; j < k1; ++j) {
      v4i q = *(const v4i*)(out16 + (t * k1 + j) * H + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[2 * i] += bf16_bits_to_f32((uint32_t)q[i] & 0xFFFFu);
        s[2 * i + 1] += bf16_bits_to_f32((uint32_t)q[i] >> 16);
      }
    }
  } else {
    const float* out32 = (const float*)out;
    const v4f* p = (const v4f*)(out32 + t * H + c);
    v4f a = p[0], b = p[1];
    s[0] = a[0]; s[1] = a[1]; s[2] = a[2]; s[3] = a[3];
    s[4] = b[0]; s[5] = b[1]; s[6] = b[2]; s[7] = b[3];
  }
  v4i o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = (int)(f32_to_bf16_bits(s[2 * i]) | (f32_to_bf16_bits(s[2 * i + 1]) << 16));
  *(v4i*)(y + t * H + c) = o;
}

}  // namespace

hipError_t launch_finalize(const void* out, int T, int H, int k1, int combine, uint16_t* y,
                           hipStream_t st) {
  size_t n = (size_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (combine == 1) hipLaunchKernelGGL(k_finalize<1>, grid, block, 0, st, out, T, H, k1, y);
  else if (combine == 3) hipLaunchKernelGGL(k_finalize<3>, grid, block, 0, st, out, T, H, k1, y);
  else hipLaunchKernelGGL(k_finalize<2>, grid, block, 0, st, out, T, H, k1, y);
  return hipGetLastError();
}

}  // namespace mxmoe
