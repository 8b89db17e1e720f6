// Fused front of the block: routing, the sort and the activation quantisation in as few launches
// as the batch allows. Launch count matters at decode sizes, where every kernel node costs a few
// microseconds ("Ling-3.0-flash: Tối ưu hóa độ trễ giải mã lên 54% trên 4 GPU Blackwell",
// "Hai loại thời gian nhàn rỗi": hundreds of 1.5-6 us kernel nodes at batch 1).
//   up to 32 tokens (and S <= 4096): one launch; workgroup 0 routes every token (each wave takes
//     at most two, back to back) into LDS and sorts the slots there (up to 16 slots, each wave
//     derives the layout in registers), the other workgroups quantise x (and clear the atomic
//     accumulator when that combine is used).
//   more tokens: one launch routes (one wave per token, 16 per workgroup) and quantises, then the
//     sort: one workgroup up to 4096 slots, the three-pass sort beyond.
//   slot-order plan (no sorted layout): the routing and quantising launch alone.
#include "align_dev.h"
#include "device.h"
#include "kernels.h"
#include "quant_dev.h"
#include "route_dev.h"

namespace mxmoe {

namespace {

constexpr int kThreads = 1024;

template <bool F32>
__global__ __launch_bounds__(kThreads) void k_prologue_small(PrologueArgs a) {
  if (blockIdx.x == 0) {
    __shared__ AlignSmem sm;
    __shared__ int32_t ids_lds[kAlignSmallMaxSlots];
    __shared__ float w_lds[kAlignTinyMaxSlots];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int S = a.T * (a.top_k + 1);
    const bool tiny = S <= kAlignTinyMaxSlots;
    for (int i = threadIdx.x; i < a.n_cnt; i += kThreads) a.zero_cnt[i] = 0;
    route_tokens_any<F32>(a.logits, wave, kThreads / 64, a.T, a.E, a.top_k, lane, a.ids, a.w,
                          ids_lds, tiny ? w_lds : nullptr);
    __syncthreads();
    if (tiny) {  // every wave derives the few slots' layout and writes its share
      align_tiny(ids_lds, w_lds, S, a.E + 1, a.block_m, a.cap, a.out, wave, kThreads / 64);
      return;
    }
    align_small_body(ids_lds, S, a.E + 1, a.block_m, a.cap, a.out, sm);
    return;
  }
  const size_t g = (size_t)(blockIdx.x - 1) * kThreads + threadIdx.x;
  const size_t blk = g >> 2;  // four lanes per block
  const int nbk = a.H / 32;
  if (blk >= (size_t)a.T * nbk) return;
  const size_t t = blk / nbk;
  quant_act_part(a.x, t, (int)(blk - t * nbk), (int)(g & 3), a.H, a.xq, a.xs, a.srs, a.a4, a.zero_out);
}

// Weight prefetch (prefetch workgroup pb of the launch, on XCD blockIdx % 8 like every workgroup
// of a launch): the first pf_steps K-steps of the weights and scales of each slot-order gate_up
// unit that XCD will run, as direct LDS loads into a scratch area (nothing waits for them but the
// workgroup's end). A unit's K-steps are contiguous in the prepacked layout.
__device__ __forceinline__ void prefetch_gate_up(const PrologueArgs& a, int pb) {
  __shared__ __attribute__((aligned(16))) uint8_t sink[(kThreads / 64) * 1024];
  constexpr int kWaves = kThreads / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int x = blockIdx.x & 7, part = pb >> 3;
  const int total = a.pf_chunks * a.pf_nb;
  const int per_xcd = (total + 7) >> 3;
  const int u0 = x * per_xcd, u1 = u0 + per_xcd < total ? u0 + per_xcd : total;
  const int pieces = a.pf_steps * a.pf_step_bytes / 1024;  // 1 KiB weight loads per unit
  const int per_unit = pieces + a.pf_steps;                // and a 256-byte scale load per step
  const int nw = a.pf_wgs * kWaves;
  const uint32_t lds =
      (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)sink + 1024u * wave;
  for (int i = part * kWaves + wave; i < (u1 - u0) * per_unit; i += nw) {
    const int u = u0 + i / per_unit, q = i - (i / per_unit) * per_unit;
    const int chunk = u / a.pf_nb, blk = u - chunk * a.pf_nb;
    const int e = blk < a.E ? blk : a.E;
    if (q < pieces) {
      const v4i r = rsrc_words(a.pf_w + (size_t)e * a.pf_wbytes, (uint32_t)a.pf_wbytes);
      lds_load16(r, lds, 16u * lane, chunk * a.pf_nks * a.pf_step_bytes + q * 1024);
    } else {
      const v4i r = rsrc_words(a.pf_ws + (size_t)e * a.pf_sbytes, (uint32_t)a.pf_sbytes);
      lds_load4(r, lds, 4u * lane, (chunk * a.pf_nks + (q - pieces)) * 256);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Larger batches: workgroups [0, n_route) route 16 tokens each; the next n_quant quantise /
// clear; any after them prefetch gate_up weights into L2.
template <bool F32>
__global__ __launch_bounds__(kThreads) void k_route_quant(PrologueArgs a, int n_route, int n_quant) {
  if ((int)blockIdx.x >= n_route + n_quant) {
    prefetch_gate_up(a, (int)blockIdx.x - n_route - n_quant);
    return;
  }
  if ((int)blockIdx.x < n_route) {
    if (blockIdx.x == 0)
      for (int i = threadIdx.x; i < a.n_cnt; i += kThreads) a.zero_cnt[i] = 0;
    const int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (t < a.T)
      route_tokens_any<F32>(a.logits, t, a.T, a.T, a.E, a.top_k, threadIdx.x & 63, a.ids, a.w,
                            nullptr);
    return;
  }
  // grid-stride over the blocks (four lanes per block; a quad's lanes share every iteration)
  const int nbk = a.H / 32;
  const size_t nblk = (size_t)a.T * nbk;
  const size_t nthr = (size_t)n_quant * kThreads;
  for (size_t g = (size_t)(blockIdx.x - n_route) * kThreads + threadIdx.x; (g >> 2) < nblk;
       g += nthr) {
    const size_t blk = g >> 2;
    const size_t t = blk / nbk;
    quant_act_part(a.x, t, (int)(blk - t * nbk), (int)(g & 3), a.H, a.xq, a.xs, a.srs, a.a4,
                   a.zero_out);
  }
}

// Quantising workgroups of the larger-batch launch: at most this many, each thread striding over
// the blocks. One thread per 8 values (3072 workgroups at 8K tokens, hidden 3072) spent more on
// workgroup dispatch than on the 75 MB it moves: prologue stage 36.3 -> 33.0 us at 8K tokens with
// 1024 workgroups (256: 35.3, 512: 33.5); no change at 4096 tokens, hidden 2048.
constexpr int kQuantMaxWgs = 1024;

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, bool logits_f32, void* align_scratch,
                           hipStream_t st) {
  const int S = a.T * (a.top_k + 1);
  const bool work = a.xq || a.zero_out;
  const int nq = work ? (int)(((size_t)a.T * (a.H / 32) * 4 + kThreads - 1) / kThreads) : 0;
  // Slot-order plan: no sort; routing spreads over workgroups (a wave per token) beside the
  // quantisation.
  // One launch while one workgroup's 16 waves route every token two at most each: a wave routes a
  // token in about 1.7 us, so at 32 tokens the fused kernel (about 11.4 us) still beats a routing
  // launch plus a sort launch (about 12.9 us with the gap between them); beyond that, routing
  // spreads over workgroups and the sort becomes a launch of its own.
  if (!a.no_sort && S <= kAlignSmallMaxSlots && a.T <= 2 * (kThreads / 64)) {
    dim3 grid(1 + nq), block(kThreads);
    if (logits_f32) hipLaunchKernelGGL(k_prologue_small<true>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(k_prologue_small<false>, grid, block, 0, st, a);
    return hipGetLastError();
  }
  const int nr = (a.T + kThreads / 64 - 1) / (kThreads / 64);
  const int nqw = nq < kQuantMaxWgs ? nq : kQuantMaxWgs;
  const int npf = a.pf_w ? 8 * a.pf_wgs : 0;
  dim3 grid(nr + nqw + npf), block(kThreads);
  if (logits_f32) hipLaunchKernelGGL(k_route_quant<true>, grid, block, 0, st, a, nr, nqw);
  else hipLaunchKernelGGL(k_route_quant<false>, grid, block, 0, st, a, nr, nqw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.no_sort) return e;
  return launch_align(a.ids, a.T, a.E, a.top_k, a.block_m, a.out, align_scratch, st);
}

}  // namespace mxmoe
