// Final rounding of the combined output to bf16. With per-slot rows (fp32 or bf16) the k+1 slot
// contributions of a token are summed here in fp32 in slot order (a fixed order, so the result is
// reproducible); with the atomic combine the token-major fp32 accumulator is only converted.
#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

// Slot rows read per batch: all loads of a batch are issued before the first add (a loop that
// adds each slot as it arrives waits one memory latency per slot).
constexpr int kBatch = 9;

// One thread per 8 consecutive output columns.
template <int COMBINE, bool NT>
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
    for (int j0 = 0; j0 < k1; j0 += kBatch) {  // a batch of slot rows in flight, then the adds
      v4f a[kBatch], b[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {  // indices past the last slot re-read it (added as zero)
        const v4f* p = (const v4f*)(out32 + (t * k1 + min(j0 + q, k1 - 1)) * H + c);
        a[q] = p[0];
        b[q] = p[1];
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const float on = j0 + q < k1 ? 1.f : 0.f;
        s[0] += on * a[q][0]; s[1] += on * a[q][1]; s[2] += on * a[q][2]; s[3] += on * a[q][3];
        s[4] += on * b[q][0]; s[5] += on * b[q][1]; s[6] += on * b[q][2]; s[7] += on * b[q][3];
      }
    }
  } else if (COMBINE == 3) {
    const uint16_t* out16 = (const uint16_t*)out;
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.f;
    for (int j0 = 0; j0 < k1; j0 += kBatch) {  // a batch of slot rows in flight, then the adds
      v4i q[kBatch];
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {  // indices past the last slot re-read it (added as zero)
        const v4i* src = (const v4i*)(out16 + (t * k1 + min(j0 + b, k1 - 1)) * H + c);
        q[b] = NT ? __builtin_nontemporal_load(src) : *src;
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        const bool on = j0 + b < k1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[2 * i] += on ? bf16_bits_to_f32((uint32_t)q[b][i] & 0xFFFFu) : 0.f;
          s[2 * i + 1] += on ? bf16_bits_to_f32((uint32_t)q[b][i] >> 16) : 0.f;
        }
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
    o[i] = (int)bf16_pair(s[2 * i], s[2 * i + 1]);
  *(v4i*)(y + t * H + c) = o;
}

}  // namespace

hipError_t launch_finalize(const void* out, int T, int H, int k1, int combine, uint16_t* y,
                           hipStream_t st) {
  size_t n = (size_t)T * (H / 8);
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  // bf16 slot rows are read once: non-temporal loads keep them from displacing cached data.
  // Measured at 8K tokens (hidden 3072, 9 slots): 105 -> 84 us (non-temporal y stores as well: 89).
  const bool nt = tuning().final_nt != 0;  // unset (-1): non-temporal
  if (combine == 1) hipLaunchKernelGGL((k_finalize<1, false>), grid, block, 0, st, out, T, H, k1, y);
  else if (combine == 3 && nt) hipLaunchKernelGGL((k_finalize<3, true>), grid, block, 0, st, out, T, H, k1, y);
  else if (combine == 3) hipLaunchKernelGGL((k_finalize<3, false>), grid, block, 0, st, out, T, H, k1, y);
  else hipLaunchKernelGGL((k_finalize<2, false>), grid, block, 0, st, out, T, H, k1, y);
  return hipGetLastError();
}

}  // namespace mxmoe
