// Token -> expert top-k router: one wavefront per token.
//
// Selection compares an order-preserving 64-bit key per expert: the logit's fp32 bit pattern mapped
// to an unsigned integer that increases with the value (-0 folded onto +0), in the high half, and
// the complemented expert index in the low half. The wave-wide maximum of that key is the
// largest logit, ties going to the lowest index — the fixed tie-break of the routing table. The
// shared expert then takes slot top_k with weight 1: the folding of the shared expert into the
// routing table described in "Lần theo điểm nghẽn: Tối ưu MiniMax M3 trên AMD Instinct MI355X"
// (shared-expert passage, Fig. 4). Weights are softmax over the selected logits (renormalised
// top-k), computed in fp32.
#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

constexpr int kMaxPerLane = kMaxExperts / 64;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = (uint32_t)__shfl_xor((int)lo, m);
  hi = (uint32_t)__shfl_xor((int)hi, m);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t order_key(uint32_t u) {
  if ((u & 0x7FFFFFFFu) == 0) u = 0;                  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t o = (uint32_t)(key >> 32);
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

template <bool F32>
__device__ void route_token(const void* logits, int t, int E, int top_k, int lane, int32_t* ids,
                            float* w) {
  const int nper = (E + 63) >> 6;
  uint64_t key[kMaxPerLane];
#pragma unroll
  for (int c = 0; c < kMaxPerLane; ++c) {
    key[c] = 0;
    int e = lane + 64 * c;
    if (c < nper && e < E) {
      uint32_t u = F32 ? ((const uint32_t*)logits)[(size_t)t * E + e]
                       : ((uint32_t)((const uint16_t*)logits)[(size_t)t * E + e] << 16);
      key[c] = ((uint64_t)order_key(u) << 32) | (uint32_t)(~(uint32_t)e);
    }
  }
  uint64_t mine = 0;  // lane j keeps the key chosen in round j
  for (int j = 0; j < top_k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int c = 0; c < kMaxPerLane; ++c) best = key[c] > best ? key[c] : best;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      uint64_t o = shfl_xor_u64(best, m);
      best = o > best ? o : best;
    }
#pragma unroll
    for (int c = 0; c < kMaxPerLane; ++c)
      if (key[c] == best) key[c] = 0;  // keys are unique: exactly one lane clears it
    if (lane == j) mine = best;
  }
  float v = key_value(mine);
  float v0 = __shfl(v, 0);
  float p = lane < top_k ? expf(v - v0) : 0.f;
  float s = p;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  int32_t* row_ids = ids + (size_t)t * (top_k + 1);
  float* row_w = w + (size_t)t * (top_k + 1);
  if (lane < top_k) {
    row_ids[lane] = (int32_t)(~(uint32_t)mine);
    row_w[lane] = p / s;
  } else if (lane == top_k) {
    row_ids[lane] = E;      // shared expert
    row_w[lane] = 1.0f;
  }
}

template <bool F32>
__global__ __launch_bounds__(256) void k_route(const void* logits, int T, int E, int top_k,
                                               int32_t* ids, float* w) {
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<F32>(logits, t, E, top_k, threadIdx.x & 63, ids, w);
}

}  // namespace

hipError_t launch_route(const void* logits, bool logits_f32, int T, int E, int top_k,
                        int32_t* ids, float* w, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  if (logits_f32)
    hipLaunchKernelGGL(k_route<true>, grid, block, 0, st, logits, T, E, top_k, ids, w);
  else
    hipLaunchKernelGGL(k_route<false>, grid, block, 0, st, logits, T, E, top_k, ids, w);
  return hipGetLastError();
}

}  // namespace mxmoe
