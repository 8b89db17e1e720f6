// moe_align: stable counting sort of the T*(k+1) routing slots into expert-contiguous,
// tile-padded runs — the work list of the grouped GEMMs (grouped MoE programs in "Lần theo điểm
// nghẽn: Tối ưu MiniMax M3 trên AMD Instinct MI355X", local-shapes passage). All counts stay on
// the device; the host only knows the capacity bound (the batch-1 decode page "Ling-3.0-flash:
// Tối ưu hóa độ trễ giải mã lên 54% trên 4 GPU Blackwell", "Hình dạng của một bước batch-1":
// fixed shapes plus padding turn counts into GPU-side indices).
//
// Stable ranks are computed 1024 slots at a time: inside a wavefront, lanes holding the same expert
// find each other with ballots (one ballot per distinct expert in the wave), and per-wave counts in
// LDS give the offset contributed by the earlier waves. Two variants:
//   small (S <= 4096): one workgroup does count, scan, padding and scatter;
//   large: per-chunk counts + in-chunk ranks, one-workgroup scan, then a scatter pass.
#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE1 = kMaxExperts + 1;  // routed + shared; the block scans take two per thread

// Mask of the lanes of this wave whose key equals this lane's key (valid lanes only).
__device__ __forceinline__ uint64_t match_peers(int key, bool valid) {
  uint64_t todo = __ballot(valid);
  uint64_t mine = 0;
  while (todo) {
    int leader = __ffsll((unsigned long long)todo) - 1;
    int kl = __shfl(key, leader);
    bool same = valid && key == kl;
    uint64_t m = __ballot(same);
    if (same) mine = m;
    todo &= ~m;
  }
  return mine;
}

// Exclusive scan over the workgroup (1024 threads, one value each); also returns the total.
__device__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    int s = s_wave[i];
    before += i < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// From per-expert counts cnt[0..E1): padded offsets off[0..E1], the touched-expert list and all
// layout outputs except the scatter of valid slots. Runs on one 1024-thread workgroup.
__device__ void layout_from_counts(const int* cnt, int* off, int E1, int S, int bm, int cap,
                                   int* s_wave, int32_t* sorted_ids, int32_t* block_expert,
                                   int32_t* num_post_pad, int32_t* expert_off, int32_t* touched,
                                   int32_t* n_touched) {
  const int t = threadIdx.x;
  const int e0 = 2 * t, e1 = 2 * t + 1;
  int c0 = e0 < E1 ? cnt[e0] : 0, c1 = e1 < E1 ? cnt[e1] : 0;
  int p0 = (c0 + bm - 1) / bm * bm, p1 = (c1 + bm - 1) / bm * bm;
  int total;
  int ex = block_excl_scan(p0 + p1, s_wave, &total);
  if (e0 < E1) off[e0] = ex;
  if (e1 < E1) off[e1] = ex + p0;
  int ntouch;
  int tx = block_excl_scan((c0 > 0) + (c1 > 0), s_wave, &ntouch);
  if (touched) {
    if (c0 > 0) touched[tx] = e0;
    if (c1 > 0) touched[tx + (c0 > 0)] = e1;
  }
  if (t == 0) {
    off[E1] = total;
    *num_post_pad = total;
    if (n_touched) *n_touched = ntouch;
  }
  __syncthreads();
  if (expert_off)
    for (int e = t; e <= E1; e += kThreads) expert_off[e] = off[e];
  // padding of each expert's run, then the unused tail
  for (int e = t; e < E1; e += kThreads)
    for (int r = off[e] + cnt[e]; r < off[e + 1]; ++r) sorted_ids[r] = S;
  for (int r = total + t; r < cap; r += kThreads) sorted_ids[r] = S;
  // expert of every tile: binary search of the tile start in off[]
  const int nb = cap / bm;
  for (int b = t; b < nb; b += kThreads) {
    int pos = b * bm, v = -1;
    if (pos < total) {
      int lo = 0, hi = E1 - 1;  // largest e with off[e] <= pos and a non-empty run
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= pos) lo = mid; else hi = mid - 1;
      }
      v = lo;
    }
    block_expert[b] = v;
  }
}

__device__ __forceinline__ int expert_of(const int32_t* ids, int f, int S, int E1) {
  if (f >= S) return -1;
  int e = ids[f];
  return (e >= 0 && e < E1) ? e : -1;  // out-of-range ids are dropped
}

// ---------------------------------------------------------------------------- small variant
__global__ __launch_bounds__(kThreads) void k_align_small(const int32_t* ids, int S, int E1,
                                                          int bm, int cap, int32_t* sorted_ids,
                                                          int32_t* block_expert,
                                                          int32_t* num_post_pad,
                                                          int32_t* expert_off, int32_t* touched,
                                                          int32_t* n_touched) {
  __shared__ int cnt[kMaxE1];
  __shared__ int off[kMaxE1 + 1];
  __shared__ int run[kMaxE1];
  __shared__ uint16_t wcnt[kWaves][kMaxE1];
  __shared__ int s_wave[kWaves];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int e = t; e < E1; e += kThreads) {
    cnt[e] = 0;
    run[e] = 0;
    for (int w = 0; w < kWaves; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  for (int f = t; f < S; f += kThreads) {
    int e = expert_of(ids, f, S, E1);
    if (e >= 0) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  layout_from_counts(cnt, off, E1, S, bm, cap, s_wave, sorted_ids, block_expert, num_post_pad,
                     expert_off, touched, n_touched);
  __syncthreads();
  for (int base = 0; base < S; base += kThreads) {
    int f = base + t;
    int e = expert_of(ids, f, S, E1);
    uint64_t peers = match_peers(e, e >= 0);
    int rank = __popcll(peers & ((1ull << lane) - 1ull));
    if (e >= 0 && rank == 0) wcnt[wave][e] = (uint16_t)__popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += wcnt[w][e];
      sorted_ids[off[e] + run[e] + before + rank] = f;
    }
    __syncthreads();
    for (int x = t; x < E1; x += kThreads) {
      int s = 0;
      for (int w = 0; w < kWaves; ++w) {
        s += wcnt[w][x];
        wcnt[w][x] = 0;
      }
      run[x] += s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------- large variant
// Pass 1: per chunk of 1024 slots, the in-chunk stable rank of every slot and the chunk's count
// per expert (hist[c * E1 + e]).
__global__ __launch_bounds__(kThreads) void k_align_count(const int32_t* ids, int S, int E1,
                                                          int32_t* rank_out, int32_t* hist) {
  __shared__ uint16_t wcnt[kWaves][kMaxE1];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int e = t; e < E1; e += kThreads)
    for (int w = 0; w < kWaves; ++w) wcnt[w][e] = 0;
  __syncthreads();
  int f = blockIdx.x * kThreads + t;
  int e = expert_of(ids, f, S, E1);
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
  for (int x = t; x < E1; x += kThreads) {
    int s = 0;
    for (int w = 0; w < kWaves; ++w) s += wcnt[w][x];
    h[x] = s;
  }
}

// Pass 2 (one workgroup): totals, padded offsets, layout outputs, and hist turned in place into the
// absolute start of each (chunk, expert) piece.
__global__ __launch_bounds__(kThreads) void k_align_scan(int32_t* hist, int nchunks, int S,
                                                         int E1, int bm, int cap,
                                                         int32_t* sorted_ids,
                                                         int32_t* block_expert,
                                                         int32_t* num_post_pad,
                                                         int32_t* expert_off, int32_t* touched,
                                                         int32_t* n_touched) {
  __shared__ int cnt[kMaxE1];
  __shared__ int off[kMaxE1 + 1];
  __shared__ int s_wave[kWaves];
  const int t = threadIdx.x;
  for (int e = t; e < E1; e += kThreads) {
    int s = 0;
    for (int c = 0; c < nchunks; ++c) {
      int v = hist[(size_t)c * E1 + e];
      hist[(size_t)c * E1 + e] = s;  // exclusive prefix over chunks
      s += v;
    }
    cnt[e] = s;
  }
  __syncthreads();
  layout_from_counts(cnt, off, E1, S, bm, cap, s_wave, sorted_ids, block_expert, num_post_pad,
                     expert_off, touched, n_touched);
  __syncthreads();
  for (int e = t; e < E1; e += kThreads) {
    int o = off[e];
    for (int c = 0; c < nchunks; ++c) hist[(size_t)c * E1 + e] += o;
  }
}

// Pass 3: sorted_ids[start(chunk, e) + rank] = f.
__global__ __launch_bounds__(kThreads) void k_align_scatter(const int32_t* ids, int S, int E1,
                                                            const int32_t* rank_in,
                                                            const int32_t* start,
                                                            int32_t* sorted_ids) {
  int f = blockIdx.x * kThreads + threadIdx.x;
  int e = expert_of(ids, f, S, E1);
  if (e < 0) return;
  sorted_ids[start[(size_t)blockIdx.x * E1 + e] + rank_in[f]] = f;
}

size_t align_cap(int S, int E1, int bm) {
  size_t cap = (size_t)S + (size_t)(E1 < S ? E1 : S) * (bm - 1);
  return (cap + bm - 1) / bm * bm;
}

}  // namespace

size_t align_scratch_bytes(int T, int E, int top_k) {
  size_t S = (size_t)T * (top_k + 1);
  if (S <= (size_t)kAlignSmallMaxSlots) return 0;
  size_t nch = (S + kAlignChunk - 1) / kAlignChunk;
  size_t rank = (S * 4 + 255) / 256 * 256;
  return rank + nch * (size_t)(E + 1) * 4;
}

hipError_t launch_align(const int32_t* ids, int T, int E, int top_k, int block_m,
                        int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_pad,
                        int32_t* expert_off, int32_t* touched, int32_t* n_touched, void* scratch,
                        hipStream_t st) {
  const int S = T * (top_k + 1), E1 = E + 1;
  const int cap = (int)align_cap(S, E1, block_m);
  if (S <= kAlignSmallMaxSlots) {
    hipLaunchKernelGGL(k_align_small, dim3(1), dim3(kThreads), 0, st, ids, S, E1, block_m, cap,
                       sorted_ids, block_expert, num_post_pad, expert_off, touched, n_touched);
    return hipGetLastError();
  }
  const int nch = (S + kAlignChunk - 1) / kAlignChunk;
  int32_t* rank = (int32_t*)scratch;
  int32_t* hist = (int32_t*)((char*)scratch + ((size_t)S * 4 + 255) / 256 * 256);
  hipLaunchKernelGGL(k_align_count, dim3(nch), dim3(kThreads), 0, st, ids, S, E1, rank, hist);
  hipLaunchKernelGGL(k_align_scan, dim3(1), dim3(kThreads), 0, st, hist, nch, S, E1, block_m, cap,
                     sorted_ids, block_expert, num_post_pad, expert_off, touched, n_touched);
  hipLaunchKernelGGL(k_align_scatter, dim3(nch), dim3(kThreads), 0, st, ids, S, E1, rank, hist,
                     sorted_ids);
  return hipGetLastError();
}

}  // namespace mxmoe
