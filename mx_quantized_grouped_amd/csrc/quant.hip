// MX quantisation (OCP Microscaling Formats v1.0 conversion rule): per block of 32 values along K,
// shared_exp = floor(log2(amax)) - emax_elem (8 for E4M3, 2 for E2M1) clamped to [-127, 127],
// scale byte = shared_exp + 127, elements rounded to nearest-even after the exact power-of-two
// scaling, saturating, sign kept. All decisions are taken on the fp32 (or exactly widened bf16)
// inputs with integer exponent arithmetic, so they are exact.
//
// Two users: activations inside the block (bf16 rows -> MXFP8 in the kernel-native layout, once per
// token; the MiniMax-M3 page "Lần theo điểm nghẽn: Tối ưu MiniMax M3 trên AMD Instinct MI355X"
// serves MXFP8 natively, results passage) and weights at load (canonical layout).
#include "device.h"
#include "kernels.h"
#include "quant_dev.h"

namespace mxmoe {

namespace {

// One thread per 32-element block of the row-major [rows, K] source.
template <bool F32, bool FP4>
__global__ __launch_bounds__(256) void k_quant_canonical(const void* src, int rows, int K,
                                                         uint8_t* codes, uint8_t* scales) {
  const int nbk = K / 32;
  size_t blk = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (blk >= (size_t)rows * nbk) return;
  size_t row = blk / nbk;
  int kb = (int)(blk - row * nbk);
  float v[32];
  load32<F32>(src, row * K + (size_t)kb * 32, v);
  int se = FP4 ? mx_shared_exp<2>(amax32(v)) : mx_shared_exp<8>(amax32(v));
  scales[blk] = (uint8_t)(se + 127);
  if (FP4) {
    uint32_t o[4];
    encode_fp4_32(v, se, o);
    *(v4i*)(codes + row * (K / 2) + (size_t)kb * 16) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  } else {
    uint32_t o[8];
    encode_fp8_32(v, se, o);
    v4i* p = (v4i*)(codes + row * K + (size_t)kb * 32);
    p[0] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    p[1] = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
  }
}

}  // namespace

hipError_t launch_quantize_canonical(const void* src, bool src_f32, int rows, int K, bool fp4,
                                     uint8_t* codes, uint8_t* scales, hipStream_t st) {
  size_t nblk = (size_t)rows * (K / 32);
  if (nblk == 0) return hipSuccess;
  dim3 grid((unsigned)((nblk + 255) / 256)), block(256);
  if (src_f32) {
    if (fp4) hipLaunchKernelGGL((k_quant_canonical<true, true>), grid, block, 0, st, src, rows, K, codes, scales);
    else hipLaunchKernelGGL((k_quant_canonical<true, false>), grid, block, 0, st, src, rows, K, codes, scales);
  } else {
    if (fp4) hipLaunchKernelGGL((k_quant_canonical<false, true>), grid, block, 0, st, src, rows, K, codes, scales);
    else hipLaunchKernelGGL((k_quant_canonical<false, false>), grid, block, 0, st, src, rows, K, codes, scales);
  }
  return hipGetLastError();
}

}  // namespace mxmoe
