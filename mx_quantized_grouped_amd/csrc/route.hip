// Token -> expert top-k router kernel (standalone entry point): one wavefront per token, four
// tokens per workgroup. The routing itself is in route_dev.h.
#include "device.h"
#include "kernels.h"
#include "route_dev.h"

namespace mxmoe {

namespace {

template <bool F32>
__global__ __launch_bounds__(256) void k_route(const void* logits, int T, int E, int top_k,
                                               int32_t* ids, float* w) {
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_tokens_any<F32>(logits, t, T, T, E, top_k, threadIdx.x & 63, ids, w, nullptr);
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
