// moe_align kernels (the counting sort itself is described in align_dev.h). Two variants:
//   tiny (S <= 16): every wave derives the layout in registers and writes its share;
//   small (S <= 4096): one workgroup does count, scan, padding and scatter;
//   large: per-chunk counts + in-chunk ranks (which also preset every slot of the layout to the
//   padding sentinel), then a placing pass in which every chunk's workgroup derives the offsets
//   from all chunk histograms and writes its valid slots and part of the tile -> expert map.
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

// Pass 2: one workgroup per chunk again. Each derives, from all the chunk histograms, the expert
// totals (hence the padded offsets, by the layout's block scan) and its own chunk's prefix per
// expert (the slots of earlier chunks), then places its slots: sorted_ids[off[e] + pre[e] + rank]
// = f (and the slot's weight into sorted_w). The workgroups also write the tile -> expert map, tile
// b belonging to the expert whose padded range [off[e], off[e + 1]) holds row b * bm (a binary
// search over the offsets in LDS), -1 past the used rows; workgroup 0 writes the layout's other
// outputs. Deriving the offsets in every workgroup replaces a one-workgroup scan launch between
// the count and the scatter (8K tokens x 129 experts: 7.1 + 4.6 us for the two).
// When the histograms fit (up to 28 Ki counts) they are first copied into LDS with coalesced loads
// all issued before the first LDS store (a plain copy loop waits for each load before issuing the
// next: one memory latency per iteration); walked in global memory, every thread's chain of loads
// costs a memory latency per count.
constexpr int kScanLdsCounts = 28 * 1024;

struct PlaceSmem {
  int cnt[kAlignMaxE1];
  int pre[kAlignMaxE1];
  int off[kAlignMaxE1 + 1];
  int s_wave[2 * kAlignWaves];
  int seg_all[kAlignThreads];
  int seg_pre[kAlignThreads];
};

// Expert totals cnt[e] and this chunk's prefix pre[e] over the chunk histograms `hist` (LDS or
// global). Threads split into (expert, segment of chunks) pairs so the histograms are walked in
// parallel. Inlined once per address space: through one pointer that may be either, every read
// became a generic (flat) load waited on one at a time.
__device__ __forceinline__ void align_chunk_sums(const int32_t* __restrict__ hist, int nchunks,
                                                 int chunk, int E1, PlaceSmem& sm) {
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
    int all = 0, before = 0;
    if (mine && ee < E1) {
#pragma unroll 8
      for (int c = c_lo; c < c_hi; ++c) {
        const int v = hist[(size_t)c * E1 + ee];
        all += v;
        before += c < chunk ? v : 0;
      }
    }
    if (pass == 0) {
      sm.seg_all[t] = all;
      sm.seg_pre[t] = before;
    } else {
      sm.cnt[ee] = all;
      sm.pre[ee] = before;
    }
  }
  __syncthreads();
  for (int x = t; x < E1 && x < kAlignThreads; x += kAlignThreads) {
    int a = 0, b = 0;
    for (int q = 0; q < P; ++q) {
      a += sm.seg_all[q * E1 + x];
      b += sm.seg_pre[q * E1 + x];
    }
    sm.cnt[x] = a;
    sm.pre[x] = b;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kAlignThreads) void k_align_place(const int32_t* ids, int S, int E1,
                                                               int bm, int cap, int nb,
                                                               const int32_t* rank_in,
                                                               const int32_t* __restrict__ hist_g,
                                                               int nchunks, AlignOut o) {
  __shared__ PlaceSmem sm;
  __shared__ int hist_l[kScanLdsCounts];
  __shared__ int npp_local;
  const int t = threadIdx.x, c = blockIdx.x;
  const int nh = nchunks * E1;
  // this thread's slot: its loads go out first, to arrive while the histograms are summed
  const int f = c * kAlignThreads + t;
  const int e = align_expert_of(ids, f, S, E1);
  const int rank = e >= 0 ? rank_in[f] : 0;
  const float wt = (e >= 0 && o.sorted_w) ? o.topk_w[f] : 0.f;
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
    align_chunk_sums(hist_l, nchunks, c, E1, sm);
  } else {
    align_chunk_sums(hist_g, nchunks, c, E1, sm);
  }
  // offsets; only workgroup 0 writes the layout's count, offsets and touched list
  AlignOut lo = o;
  if (c != 0) {
    lo.num_post_pad = &npp_local;
    lo.expert_off = nullptr;
    lo.touched = nullptr;
    lo.n_touched = nullptr;
  }
  align_layout_from_counts(sm.cnt, sm.off, E1, S, bm, cap, sm.s_wave, lo, nullptr, false);
  if (e >= 0) {
    const int pos = sm.off[e] + sm.pre[e] + rank;
    o.sorted_ids[pos] = f;
    if (o.sorted_w) o.sorted_w[pos] = wt;
  }
  const int total = sm.off[E1];
  for (int b = c * kAlignThreads + t; b < nb; b += gridDim.x * kAlignThreads) {
    const int r = b * bm;
    int be = -1;
    if (r < total) {
      int lo2 = 0, hi = E1 - 1;  // largest e with off[e] <= r (empty experts share offsets)
      while (lo2 < hi) {
        const int mid = (lo2 + hi + 1) >> 1;
        if (sm.off[mid] <= r) lo2 = mid;
        else hi = mid - 1;
      }
      be = lo2;
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
  return rank + hist;  // in-chunk ranks, chunk histograms
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
  int32_t* hist = (int32_t*)((char*)scratch + ((size_t)S * 4 + 255) / 256 * 256);
  hipLaunchKernelGGL(k_align_count, dim3(nch), dim3(kAlignThreads), 0, st, ids, S, E1, cap, rank,
                     hist, o);
  hipLaunchKernelGGL(k_align_place, dim3(nch), dim3(kAlignThreads), 0, st, ids, S, E1, block_m,
                     cap, cap / block_m, rank, hist, nch, o);
  return hipGetLastError();
}

}  // namespace mxmoe
