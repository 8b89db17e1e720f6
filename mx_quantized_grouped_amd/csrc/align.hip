// moe_align kernels (the counting sort itself is described in align_dev.h). Two variants:
//   tiny (S <= 16): every wave derives the layout in registers and writes its share;
//   small (S <= 4096): one workgroup does count, scan, padding and scatter;
//   large: per-chunk counts + in-chunk ranks (which also preset every slot of the layout to the
//   padding sentinel), a one-workgroup scan of the offsets, then a scatter pass that writes the
//   valid slots and the tile -> expert map. Only the offsets go through the single workgroup: its
//   padding and tile fill took 8 of the 14 us of the 8K-token sort.
#include "align_dev.h"
#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

__global__ __launch_bounds__(kAlignThreads) void k_align_small(const int32_t* ids, int S, int E1,
                                                               int bm, int cap, AlignOut o) {
  if (S <= kAlignTinyMaxSlots) {
    align_tiny(ids, o.topk_w, S, E1, bm, cap, o, threadIdx.x >> 6, kAlignWaves);
    return;
  }
  __shared__ AlignSmem sm;
  align_small_body(ids, S, E1, bm, cap, o, sm);
}

// Pass 1: per chunk of 1024 slots, the in-chunk stable rank of every slot and the chunk's count
// per expert (hist[c * E1 + e]); the workgroups also preset all cap layout slots to the padding
// sentinel S (weight 0), consecutive threads on consecutive slots. The scatter pass overwrites
// the valid ones.
__global__ __launch_bounds__(kAlignThreads) void k_align_count(const int32_t* ids, int S, int E1,
                                                               int cap, int32_t* rank_out,
                                                               int32_t* hist, AlignOut o) {
  __shared__ uint16_t wcnt[kAlignWaves][kAlignMaxE1];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int r = blockIdx.x * kAlignThreads + t; r < cap; r += gridDim.x * kAlignThreads) {
    o.sorted_ids[r] = S;
    if (o.sorted_w) o.sorted_w[r] = 0.f;
  }
  for (int e = t; e < E1; e += kAlignThreads)
    for (int w = 0; w < kAlignWaves; ++w) wcnt[w][e] = 0;
  __syncthreads();
  int f = blockIdx.x * kAlignThreads + t;
  int e = align_expert_of(ids, f, S, E1);
  uint64_t peers = match_peers(e, e >= 0);
  int rank = __popcll(peers & ((1ull << lane) - 1ull));
  if (e >= 0 && rank == 0) wcnt[wave][e] = (uint16_t)__popcll(peers);
  __syncthreads();
  if (e >= 0) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wcnt[w][e];
    rank_out[f] = before + rank;
  }
  int32_t* h = hist + (size_t)blockIdx.x * E1;
  for (int x = t; x < E1; x += kAlignThreads) {
    int s = 0;
    for (int w = 0; w < kAlignWaves; ++w) s += wcnt[w][x];
    h[x] = s;
  }
}

// Pass 2 (one workgroup): totals, padded offsets and layout outputs; start[c * E1 + e] becomes the
// absolute start of the (chunk c, expert e) piece. Threads split into (expert, segment of chunks)
// pairs so the chunk histograms are walked in parallel. When the histograms fit (up to 28 Ki
// counts), they are first copied into LDS with coalesced loads all issued before the first LDS
// store (a plain copy loop waits for each load before issuing the next: one memory latency per
// iteration; batches of 8 per thread still took three memory latencies for 4096 tokens over 512
// experts); walked in global memory, the per-thread chain of loads made this pass take 16 us for
// an 8K-token batch.
constexpr int kScanLdsCounts = 28 * 1024;

// The scan proper over the chunk histograms `hist` (LDS or global). It is inlined once per
// address space: through one pointer that may be either, every read of the walks below became a
// generic (flat) load waited on one at a time, ~70 of them per thread for 4096 tokens over 512
// experts.
__device__ __forceinline__ void align_scan_body(const int32_t* __restrict__ hist,
                                                int32_t* __restrict__ start,
                                                int32_t* __restrict__ offs, int nchunks, int S,
                                                int E1, int bm, int cap, const AlignOut& o,
                                                int* cnt, int* off, int* s_wave, int* seg_sum) {
  const int t = threadIdx.x;
  const int P = E1 >= kAlignThreads ? 1 : kAlignThreads / E1;  // segments per expert
  const int seg = (nchunks + P - 1) / P;
  const int part = t / E1, e = t - part * E1;
  const bool mine = part < P;
  int c_lo = 0, c_hi = 0;
  if (mine) {
    c_lo = part * seg;
    c_hi = min(nchunks, c_lo + seg);
  }
  // experts beyond the first 1024 (E1 > 1024) are summed by a second pass of the same threads
  for (int ee = e, pass = 0; pass < 2; ++pass, ee += kAlignThreads) {
    if (pass == 1 && (P != 1 || ee >= E1)) break;
    int sum = 0;
    if (mine && ee < E1) {
#pragma unroll 8
      for (int c = c_lo; c < c_hi; ++c) sum += hist[(size_t)c * E1 + ee];
    }
    if (pass == 0) seg_sum[t] = sum;
    else cnt[ee] = sum;
  }
  __syncthreads();
  for (int x = t; x < E1 && x < kAlignThreads; x += kAlignThreads) {
    if (P == 1) { cnt[x] = seg_sum[x]; continue; }
    int s2 = 0;
    for (int q = 0; q < P; ++q) {
      int v = seg_sum[q * E1 + x];
      seg_sum[q * E1 + x] = s2;  // exclusive prefix over segments
      s2 += v;
    }
    cnt[x] = s2;
  }
  __syncthreads();
  align_layout_from_counts(cnt, off, E1, S, bm, cap, s_wave, o, nullptr, false);
  for (int x = t; x <= E1; x += kAlignThreads) offs[x] = off[x];
  __syncthreads();
  for (int ee = e, pass = 0; pass < 2; ++pass, ee += kAlignThreads) {
    if (pass == 1 && (P != 1 || ee >= E1)) break;
    if (!mine || ee >= E1) continue;
    int run = off[ee] + (P == 1 ? 0 : seg_sum[t]);
#pragma unroll 8
    for (int c = c_lo; c < c_hi; ++c) {
      start[(size_t)c * E1 + ee] = run;
      run += hist[(size_t)c * E1 + ee];
    }
  }
}

__global__ __launch_bounds__(kAlignThreads) void k_align_scan(const int32_t* __restrict__ hist_g,
                                                              int32_t* __restrict__ start,
                                                              int32_t* __restrict__ offs,
                                                              int nchunks, int S, int E1, int bm,
                                                              int cap, AlignOut o) {
  __shared__ int cnt[kAlignMaxE1];
  __shared__ int off[kAlignMaxE1 + 1];
  __shared__ int s_wave[2 * kAlignWaves];
  __shared__ int seg_sum[kAlignThreads];
  __shared__ int hist_l[kScanLdsCounts];
  const int t = threadIdx.x;
  const int nh = nchunks * E1;
  if (nh <= kScanLdsCounts) {
    constexpr int kB = kScanLdsCounts / kAlignThreads;  // every load in one batch
    for (int base = t; base < nh; base += kB * kAlignThreads) {
      int v[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int i = base + j * kAlignThreads;
        v[j] = i < nh ? hist_g[i] : 0;
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int i = base + j * kAlignThreads;
        if (i < nh) hist_l[i] = v[j];
      }
    }
    __syncthreads();
    align_scan_body(hist_l, start, offs, nchunks, S, E1, bm, cap, o, cnt, off, s_wave, seg_sum);
  } else {
    align_scan_body(hist_g, start, offs, nchunks, S, E1, bm, cap, o, cnt, off, s_wave, seg_sum);
  }
}

// Pass 3: sorted_ids[start(chunk, e) + rank] = f (and the slot's weight into sorted_w); the
// workgroups also write the tile -> expert map, tile b belonging to the expert whose padded range
// [offs[e], offs[e + 1]) holds row b * bm (a binary search over the offsets in LDS), -1 past the
// used rows.
__global__ __launch_bounds__(kAlignThreads) void k_align_scatter(const int32_t* ids, int S, int E1,
                                                                 int bm, int nb,
                                                                 const int32_t* rank_in,
                                                                 const int32_t* start,
                                                                 const int32_t* offs, AlignOut o) {
  __shared__ int off[kAlignMaxE1 + 1];
  const int t = threadIdx.x;
  const int f = blockIdx.x * kAlignThreads + t;
  const int e = align_expert_of(ids, f, S, E1);
  if (e >= 0) {
    const int pos = start[(size_t)blockIdx.x * E1 + e] + rank_in[f];
    o.sorted_ids[pos] = f;
    if (o.sorted_w) o.sorted_w[pos] = o.topk_w[f];
  }
  if (blockIdx.x * kAlignThreads >= nb) return;  // workgroup-uniform: no tiles left for it
  for (int x = t; x <= E1; x += kAlignThreads) off[x] = offs[x];
  __syncthreads();
  const int total = off[E1];
  for (int b = blockIdx.x * kAlignThreads + t; b < nb; b += gridDim.x * kAlignThreads) {
    const int r = b * bm;
    int be = -1;
    if (r < total) {
      int lo = 0, hi = E1 - 1;  // largest e with off[e] <= r (empty experts share offsets)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= r) lo = mid;
        else hi = mid - 1;
      }
      be = lo;
    }
    o.block_expert[b] = be;
  }
}

}  // namespace

size_t align_cap(int S, int E1, int bm) {
  size_t cap = (size_t)S + (size_t)(E1 < S ? E1 : S) * (bm - 1);
  return (cap + bm - 1) / bm * bm;
}

size_t align_scratch_bytes(int T, int E, int top_k) {
  size_t S = (size_t)T * (top_k + 1);
  if (S <= (size_t)kAlignSmallMaxSlots) return 0;
  size_t nch = (S + kAlignChunk - 1) / kAlignChunk;
  size_t rank = (S * 4 + 255) / 256 * 256;
  size_t hist = (nch * (size_t)(E + 1) * 4 + 255) / 256 * 256;
  size_t offs = ((size_t)(E + 2) * 4 + 255) / 256 * 256;
  return rank + 2 * hist + offs;  // rank, chunk histograms, chunk starts, expert offsets
}

hipError_t launch_align(const int32_t* ids, int T, int E, int top_k, int block_m,
                        const AlignOut& o, void* scratch, hipStream_t st) {
  const int S = T * (top_k + 1), E1 = E + 1;
  const int cap = (int)align_cap(S, E1, block_m);
  if (S <= kAlignSmallMaxSlots) {
    hipLaunchKernelGGL(k_align_small, dim3(1), dim3(kAlignThreads), 0, st, ids, S, E1, block_m,
                       cap, o);
    return hipGetLastError();
  }
  const int nch = (S + kAlignChunk - 1) / kAlignChunk;
  int32_t* rank = (int32_t*)scratch;
  const size_t hist_bytes = ((size_t)nch * E1 * 4 + 255) / 256 * 256;
  int32_t* hist = (int32_t*)((char*)scratch + ((size_t)S * 4 + 255) / 256 * 256);
  int32_t* start = (int32_t*)((char*)hist + hist_bytes);
  int32_t* offs = (int32_t*)((char*)start + hist_bytes);
  hipLaunchKernelGGL(k_align_count, dim3(nch), dim3(kAlignThreads), 0, st, ids, S, E1, cap, rank,
                     hist, o);
  hipLaunchKernelGGL(k_align_scan, dim3(1), dim3(kAlignThreads), 0, st, hist, start, offs, nch, S,
                     E1, block_m, cap, o);
  hipLaunchKernelGGL(k_align_scatter, dim3(nch), dim3(kAlignThreads), 0, st, ids, S, E1, block_m,
                     cap / block_m, rank, start, offs, o);
  return hipGetLastError();
}

}  // namespace mxmoe
