// Load-time conversion of canonical expert weights into the kernel-native, fragment-major layout
// (the reordering of MXFP8 weights and scales moved to model load in "Lần theo điểm nghẽn: Tối ưu
// MiniMax M3 trên AMD Instinct MI355X", shared-expert/AITER passage).
//
// A fragment is one 16-row x 128-K tile of an expert's weight matrix, stored exactly in the order a
// wavefront's lanes consume it as the B operand of one gfx950 MFMA, so each wave load of a fragment
// is a contiguous 1 KiB:
//   MXFP8 (2 KiB): [half h][lane l][16 B]; lane l = n + 16 g holds row n, K = 16g..16g+15 (h = 0)
//                  and 64+16g..64+16g+15 (h = 1) of the tile — the operand order of
//                  v_mfma_scale_f32_16x16x128_f8f6f4 for 8-bit elements.
//   MXFP4 (1 KiB): [lane l][16 B]; lane l holds row n, K = 32g..32g+31, low nibble first.
//   bf16  (4 KiB): [sub-step s][lane l][16 B]; lane l holds row n, K = 32s+8g..32s+8g+7 (the
//                  v_mfma_f32_16x16x32_bf16 operand order, four per 128-K step).
// Fragments of an expert are ordered [group of four tiles q][K-step ks][tile 4q + f]: the four
// fragments one wave multiplies in a K-step are adjacent, so a wave streams its weights as one
// contiguous range. For W13 the tiles alternate gate and up: tile 2p holds gate rows 16p..16p+15
// and tile 2p+1 up rows I+16p..I+16p+15, so one wave holds matching gate and up columns for the
// SwiGLU epilogue. For W2 the four tiles of a group interleave their rows: tile 4q + f holds rows
// 64q + 4n + f (n = 0..15), so the four fragments a wave multiplies give each lane four adjacent
// output columns, stored as one piece by the down epilogues.
// Scales: per (expert, group of four tiles q, K-step ks) 64 dwords; byte f of lane l = n + 16g is
// the scale of row n of tile 4q + f for K-block 4ks + g. One dword load per lane and K-step serves
// the four fragments a wave multiplies (the MFMA's scale operand selects byte f). K is zero-padded
// to a multiple of 128 (scale byte 127 there). The tile count of an expert is a multiple of 4.
#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

__device__ __forceinline__ int src_row(int nt, int n, bool w13, int I) {
  if (!w13) return (nt >> 2) * 64 + 4 * n + (nt & 3);
  int p = nt >> 1;
  return (nt & 1) ? I + p * 16 + n : p * 16 + n;
}

// One thread per 16-byte chunk of the prepacked codes.
template <int WF>
__global__ __launch_bounds__(256) void k_prepack_codes(const uint8_t* src, uint8_t* dst, int E1,
                                                       int N, int K, bool w13, int I) {
  constexpr int FB = WF == WF_FP8 ? 2048 : (WF == WF_FP4 ? 1024 : 4096);
  constexpr int CH = FB / 16;  // chunks per fragment
  const int NT = N / 16, NKS = (K + KSTEP - 1) / KSTEP;
  size_t chunk = (size_t)blockIdx.x * 256 + threadIdx.x;
  size_t total = (size_t)E1 * NT * NKS * CH;
  if (chunk >= total) return;
  int c = (int)(chunk % CH);
  size_t frag = chunk / CH;
  const int f = (int)(frag & 3);
  size_t r = frag >> 2;
  int ks = (int)(r % NKS);
  size_t eq = r / NKS;
  const int NQ = NT / 4;
  int nt = 4 * (int)(eq % NQ) + f;
  size_t e = eq / NQ;
  int l, kin;  // lane, first K index (within the step) of this chunk
  if (WF == WF_FP8) {
    int h = c >> 6;
    l = c & 63;
    kin = 64 * h + 16 * (l >> 4);
  } else if (WF == WF_FP4) {
    l = c;
    kin = 32 * (l >> 4);
  } else {
    int s = c >> 6;
    l = c & 63;
    kin = 32 * s + 8 * (l >> 4);
  }
  int row = src_row(nt, l & 15, w13, I);
  int k = ks * KSTEP + kin;
  v4i val = v4i{0, 0, 0, 0};
  if (k < K) {
    size_t rb = (size_t)e * N + row;
    if (WF == WF_FP8) val = *(const v4i*)(src + rb * K + k);
    else if (WF == WF_FP4) val = *(const v4i*)(src + rb * (K / 2) + k / 2);
    else val = *(const v4i*)(src + (rb * K + k) * 2);
  }
  *(v4i*)(dst + chunk * 16) = val;
}

// One thread per prepacked scale dword.
__global__ __launch_bounds__(256) void k_prepack_scales(const uint8_t* src, uint32_t* dst, int E1,
                                                        int N, int K, bool w13, int I) {
  const int NQ = N / 64, NKS = (K + KSTEP - 1) / KSTEP, KB = K / 32;
  size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  size_t total = (size_t)E1 * NQ * NKS * 64;
  if (idx >= total) return;
  int l = (int)(idx & 63);
  size_t r = idx >> 6;
  int ks = (int)(r % NKS);
  size_t eq = r / NKS;
  int q = (int)(eq % NQ);
  size_t e = eq / NQ;
  const int kb = 4 * ks + (l >> 4);
  uint32_t v = 0;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    int row = src_row(4 * q + f, l & 15, w13, I);
    uint32_t b = kb < KB ? src[((size_t)e * N + row) * KB + kb] : 127u;
    v |= b << (8 * f);
  }
  dst[idx] = v;
}

}  // namespace

size_t prepack_code_bytes(const PrepackDims& d) {
  size_t FB = d.wf == WF_FP8 ? 2048 : (d.wf == WF_FP4 ? 1024 : 4096);
  size_t NKS = (d.K + KSTEP - 1) / KSTEP;
  return (size_t)d.E1 * (d.N / 16) * NKS * FB;
}

size_t prepack_scale_bytes(const PrepackDims& d) {
  if (d.wf == WF_BF16) return 0;
  size_t NKS = (d.K + KSTEP - 1) / KSTEP;
  return (size_t)d.E1 * (d.N / 64) * NKS * 256;
}

hipError_t launch_prepack(const PrepackDims& d, const void* codes, const uint8_t* scales,
                          void* codes_p, void* scales_p, hipStream_t st) {
  size_t chunks = prepack_code_bytes(d) / 16;
  dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
  const uint8_t* src = (const uint8_t*)codes;
  uint8_t* dst = (uint8_t*)codes_p;
  if (d.wf == WF_FP8)
    hipLaunchKernelGGL(k_prepack_codes<WF_FP8>, grid, block, 0, st, src, dst, d.E1, d.N, d.K, d.w13, d.I);
  else if (d.wf == WF_FP4)
    hipLaunchKernelGGL(k_prepack_codes<WF_FP4>, grid, block, 0, st, src, dst, d.E1, d.N, d.K, d.w13, d.I);
  else
    hipLaunchKernelGGL(k_prepack_codes<WF_BF16>, grid, block, 0, st, src, dst, d.E1, d.N, d.K, d.w13, d.I);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || d.wf == WF_BF16) return err;
  size_t words = prepack_scale_bytes(d) / 4;
  hipLaunchKernelGGL(k_prepack_scales, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, st,
                     scales, (uint32_t*)scales_p, d.E1, d.N, d.K, d.w13, d.I);
  return hipGetLastError();
}

}  // namespace mxmoe
