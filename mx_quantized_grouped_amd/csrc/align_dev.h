// Device side of moe_align: stable counting sort of the T*(k+1) routing slots into
// expert-contiguous, tile-padded runs — the work list of the grouped GEMMs (grouped MoE programs
// in "Lần theo điểm nghẽn: Tối ưu MiniMax M3 trên AMD Instinct MI355X", local-shapes passage). All
// counts stay on the device; the host only knows the capacity bound (the batch-1 decode page
// "Ling-3.0-flash: Tối ưu hóa độ trễ giải mã lên 54% trên 4 GPU Blackwell", "Hình dạng của một
// bước batch-1": fixed shapes plus padding turn counts into GPU-side indices).
//
// Stable ranks are computed 1024 slots at a time: inside a wavefront, lanes holding the same expert
// find each other with ballots (one ballot per distinct expert in the wave), and per-wave counts in
// LDS give the offset contributed by the earlier waves.
#pragma once
#include "device.h"
#include "kernels.h"

namespace mxmoe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kAlignMaxE1 = kMaxExperts + 1;  // routed + shared; the block scans take two per thread

// Small layouts get their padding and tile lists from a tile -> expert map in LDS, written with
// coalesced passes over every slot and tile (see align_layout_from_counts).
constexpr int kTileMapMax = 4096;       // tiles
constexpr int kParallelFillMax = 16384; // slots

// LDS of the single-workgroup sort. Per-wave counts (ballot variant) or one bit per slot per
// expert (bitmap variant) share the same space.
constexpr int kAlignBitmapWords = kAlignWaves * kAlignMaxE1 * 2 / 8;
struct AlignSmem {
  int cnt[kAlignMaxE1];
  int off[kAlignMaxE1 + 1];
  int run[kAlignMaxE1];
  union {
    uint16_t wcnt[kAlignWaves][kAlignMaxE1];
    unsigned long long bits[kAlignBitmapWords];
  };
  int s_wave[2 * kAlignWaves];
  int16_t tile_e[kTileMapMax];
};

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

// Inclusive scan over the 64 lanes of the wave with DPP: shifts by 1, 2, 4, 8 inside each 16-lane
// row (lanes shifted in from outside the row add 0), then the row totals are carried by two row
// broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive scan over the 1024-thread workgroup (one value each); also returns the total.
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kAlignWaves; ++i) {
    int s = s_wave[i];
    before += i < wave ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Exclusive scans of two values at once over the 1024-thread workgroup (one barrier for both):
// ea / eb the exclusive prefixes, ta / tb the totals. s_wave holds 2 * kAlignWaves ints; the caller
// puts a barrier between this scan and the next use of s_wave.
__device__ __forceinline__ void block_excl_scan2(int a, int b, int* s_wave, int* ea, int* eb,
                                                 int* ta, int* tb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int xa = wave_incl_scan(a), xb = wave_incl_scan(b);
  if (lane == 63) {
    s_wave[wave] = xa;
    s_wave[kAlignWaves + wave] = xb;
  }
  __syncthreads();
  int ba = 0, bb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < kAlignWaves; ++i) {
    const int va = s_wave[i], vb = s_wave[kAlignWaves + i];
    ba += i < wave ? va : 0;
    bb += i < wave ? vb : 0;
    sa += va;
    sb += vb;
  }
  *ea = ba + xa - a;
  *eb = bb + xb - b;
  *ta = sa;
  *tb = sb;
}

__device__ __forceinline__ int align_expert_of(const int32_t* ids, int f, int S, int E1) {
  if (f >= S) return -1;
  int e = ids[f];
  return (e >= 0 && e < E1) ? e : -1;  // out-of-range ids are dropped
}

// From per-expert counts cnt[0..E1): padded offsets off[0..E1], the touched-expert list and all
// layout outputs except the scatter of valid slots. Called by the whole 1024-thread workgroup.
// tile_e: LDS room for kTileMapMax tile -> expert entries, or null. With fill false, the padding
// slots and the tile -> expert map are left to the caller (the multi-workgroup sort writes them
// from its parallel passes).
// align_layout_core takes this thread's two counts (experts 2t and 2t + 1) in registers; cnt (in
// LDS, all E1 counts) is read only by the padding fill, after the barriers inside. On return off is
// complete and visible to the workgroup.
inline __device__ void align_layout_core(int c0, int c1, const int* cnt, int* off, int E1, int S,
                                         int bm, int cap, int* s_wave, const AlignOut& o,
                                         int16_t* tile_e, bool fill);

inline __device__ void align_layout_from_counts(const int* cnt, int* off, int E1, int S, int bm,
                                                int cap, int* s_wave, const AlignOut& o,
                                                int16_t* tile_e, bool fill = true) {
  const int e0 = 2 * threadIdx.x, e1 = e0 + 1;
  align_layout_core(e0 < E1 ? cnt[e0] : 0, e1 < E1 ? cnt[e1] : 0, cnt, off, E1, S, bm, cap,
                    s_wave, o, tile_e, fill);
}

inline __device__ void align_layout_core(int c0, int c1, const int* cnt, int* off, int E1, int S,
                                         int bm, int cap, int* s_wave, const AlignOut& o,
                                         int16_t* tile_e, bool fill) {
  const int t = threadIdx.x;
  const int e0 = 2 * t, e1 = 2 * t + 1;
  int p0 = (c0 + bm - 1) / bm * bm, p1 = (c1 + bm - 1) / bm * bm;
  int ex, tx, total, ntouch;
  block_excl_scan2(p0 + p1, (c0 > 0) + (c1 > 0), s_wave, &ex, &tx, &total, &ntouch);
  if (e0 < E1) off[e0] = ex;
  if (e1 < E1) off[e1] = ex + p0;
  if (o.touched) {
    if (c0 > 0) o.touched[tx] = e0;
    if (c1 > 0) o.touched[tx + (c0 > 0)] = e1;
  }
  if (t == 0) {
    off[E1] = total;
    *o.num_post_pad = total;
    if (o.n_touched) *o.n_touched = ntouch;
  }
  __syncthreads();
  if (o.expert_off)
    for (int e = t; e <= E1; e += kAlignThreads) o.expert_off[e] = off[e];
  if (!fill) return;
  const int nb = cap / bm;
  if (tile_e && nb <= kTileMapMax && cap <= kParallelFillMax) {
    // Small layout: the tile -> expert map goes to LDS, then every tile and slot is visited by
    // consecutive threads, so each store instruction writes consecutive entries (a thread per
    // expert, each writing its own padding, made every store touch 64 cache lines: 3 us of the
    // 6 us sort of a 32-token batch).
    for (int e = t; e < E1; e += kAlignThreads)
      for (int b = off[e] / bm; b < off[e + 1] / bm; ++b) tile_e[b] = (int16_t)e;
    __syncthreads();
    for (int b = t; b < nb; b += kAlignThreads) o.block_expert[b] = b * bm < total ? tile_e[b] : -1;
    for (int r = t; r < cap; r += kAlignThreads) {
      bool pad = true;
      if (r < total) {
        const int e = tile_e[r / bm];
        pad = r - off[e] >= cnt[e];
      }
      if (pad) {
        o.sorted_ids[r] = S;
        if (o.sorted_w) o.sorted_w[r] = 0.f;
      }
    }
    return;
  }
  // Padding of each expert's run and the expert of each of its tiles. With tall tiles (up to 255
  // padding slots per expert) one wave takes an expert, so consecutive lanes write consecutive
  // entries: a thread per expert makes every store instruction touch 64 cache lines (~20 us for
  // the 8K-token layout at 128-row tiles). With short tiles a thread per expert is cheaper (a wave
  // walking 8 experts in turn cost 2 us more at 16-row tiles).
  if (bm > 32) {
    const int lane = t & 63;
    for (int e = t >> 6; e < E1; e += kAlignWaves) {
      const int o0 = off[e], o1 = off[e + 1];
      for (int r = o0 + cnt[e] + lane; r < o1; r += 64) {
        o.sorted_ids[r] = S;
        if (o.sorted_w) o.sorted_w[r] = 0.f;
      }
      for (int b = o0 / bm + lane; b < o1 / bm; b += 64) o.block_expert[b] = e;
    }
  } else {
    for (int e = t; e < E1; e += kAlignThreads) {
      const int o0 = off[e], o1 = off[e + 1];
      for (int r = o0 + cnt[e]; r < o1; ++r) {
        o.sorted_ids[r] = S;
        if (o.sorted_w) o.sorted_w[r] = 0.f;
      }
      for (int b = o0 / bm; b < o1 / bm; ++b) o.block_expert[b] = e;
    }
  }
  for (int r = total + t; r < cap; r += kAlignThreads) {
    o.sorted_ids[r] = S;
    if (o.sorted_w) o.sorted_w[r] = 0.f;
  }
  for (int b = total / bm + t; b < nb; b += kAlignThreads) o.block_expert[b] = -1;
}

// ---------------------------------------------------------------------------- few-slot layout
// Up to 16 slots (one token at top-8, or a few at top-2). Every wave of the workgroup derives the whole run
// structure in its own registers, one slot per lane, then writes its share of the outputs: no
// workgroup barrier and no LDS. Slot f's key is (expert << 6) | f, so the sorted order is by expert
// and, within an expert, by slot (the stable order); a slot's position in that order is the number
// of smaller keys. In sorted order the experts form runs: a run starts where the expert changes,
// the in-run rank is the distance from its first lane, and the padded offsets are an exclusive
// scan of the runs' padded sizes. The runs are compacted into lanes 0 .. nruns - 1; each output
// entry then finds its run by cross-lane reads, and consecutive lanes store consecutive entries.
// Same outputs as the workgroup sort. The serial parts (a read per slot for the ranks, per run for
// the block map and the expert offsets) grow with the slot count; measured against the workgroup
// sort (forward, 512 experts): one token 19.8 -> 18.9 us, six tokens (54 slots) 23.3 -> 25.5 us,
// so the few-slot path stops at 16. The algorithm itself is written for up to 64 slots.
constexpr int kAlignTinyMaxSlots = 16;

// v of lane src (0 <= src < 64). Cross-lane reads see only lanes that take part, so every call
// below is made by all 64 lanes (outside any lane-dependent branch), and results are selected after.
__device__ __forceinline__ int lane_read(int v, int src) {
  return __builtin_amdgcn_ds_bpermute(src << 2, v);
}

// Called by whole waves: wave `wave` of `nwaves`. ids / wsrc: the S <= 64 slots' expert ids and
// routing weights (LDS or global memory; wsrc may be null when o.sorted_w is). Out-of-range ids
// are dropped, as in the workgroup sort.
inline __device__ void align_tiny(const int32_t* ids, const float* wsrc, int S, int E1, int bm,
                                  int cap, const AlignOut& o, int wave, int nwaves) {
  const int lane = lane_id();
  const uint64_t below = (1ull << lane) - 1ull;
  const int e = lane < S ? ids[lane] : -1;
  const bool valid = e >= 0 && e < E1;
  const float wt = (o.sorted_w && lane < S) ? wsrc[lane] : 0.f;
  const uint32_t key = valid ? ((uint32_t)e << 6) | (uint32_t)lane : 0xFFFFFFFFu;
  const int nvalid = __popcll(__builtin_amdgcn_ballot_w64(valid));
  int rank = 0;
  for (int m = 0; m < S; ++m) rank += (uint32_t)__builtin_amdgcn_readlane((int)key, m) < key;
  // lane r receives the key of sorted position r; every dropped slot and every lane past S has
  // rank nvalid, so each lane below nvalid receives exactly one valid key
  const int sk = __builtin_amdgcn_ds_permute(rank << 2, (int)key);
  const bool sv = lane < nvalid;
  const int se = sv ? (int)((uint32_t)sk >> 6) : -1;
  const int prev = lane_read(se, lane > 0 ? lane - 1 : 0);
  const bool start = sv && (lane == 0 || prev != se);
  const uint64_t starts = __builtin_amdgcn_ballot_w64(start);
  const int nruns = __popcll(starts);
  // runs compacted: lane g holds run g's first sorted lane, expert, count and padded offset
  const int gi = __popcll(starts & below);
  const int dst = start ? gi : nruns + (lane - gi);  // a permutation of the lanes
  const int rfirst = __builtin_amdgcn_ds_permute(dst << 2, lane);
  const int rexp = __builtin_amdgcn_ds_permute(dst << 2, se);
  const bool rv = lane < nruns;
  const int nfirst = lane_read(rfirst, lane < 63 ? lane + 1 : 63);
  const int rnext = lane + 1 < nruns ? nfirst : nvalid;
  const int rcnt = rv ? rnext - rfirst : 0;
  const int rpad = (rcnt + bm - 1) / bm * bm;
  const int incl = wave_incl_scan(rpad);
  const int roff = incl - rpad;
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int nblk = total / bm;  // <= 64: a run of c >= 1 slots has at most c blocks
  // block b's run: the number of runs starting at or before row b * bm, less one
  int brun = -1;
  for (int g = 0; g < nruns; ++g) brun += __builtin_amdgcn_readlane(roff, g) <= lane * bm;
  const int sslot = sk & 63;  // slot id at sorted position lane
  const float swt = __int_as_float(lane_read(__float_as_int(wt), sslot));
  for (int r0 = 64 * wave; r0 < cap; r0 += 64 * nwaves) {
    const int r = r0 + lane;
    const int g = lane_read(brun, (r / bm) & 63) & 63;
    const int j = r - lane_read(roff, g);
    const int pos = (lane_read(rfirst, g) + j) & 63;
    const int sid = lane_read(sslot, pos);
    const float sw = __int_as_float(lane_read(__float_as_int(swt), pos));
    const int cnt = lane_read(rcnt, g);
    const bool slot = r < total && j < cnt;
    if (r < cap) {
      o.sorted_ids[r] = slot ? sid : S;
      if (o.sorted_w) o.sorted_w[r] = slot ? sw : 0.f;
    }
  }
  const int nb_cap = cap / bm;
  const int bexp = lane_read(rexp, brun & 63);  // expert of block lane
  for (int b0 = 64 * wave; b0 < nb_cap; b0 += 64 * nwaves) {
    const int b = b0 + lane;
    if (b < nb_cap) o.block_expert[b] = b < nblk ? bexp : -1;
  }
  if (wave == nwaves - 1) {
    if (o.touched && rv) o.touched[lane] = rexp;
    if (lane == 0) {
      *o.num_post_pad = total;
      if (o.n_touched) *o.n_touched = nruns;
    }
  }
  if (!o.expert_off) return;
  // expert_off[x] = offset of the first chosen expert >= x (total past the last one), i.e. of run
  // G(x), G(x) = the number of chosen experts below x. Entries x = lane + 64 i for this wave's
  // rounds i: G = (runs whose expert is below 64 i) + (chosen experts in word i below the lane),
  // the word's bits gathered from the runs with scalar operations.
  for (int i = wave; 64 * i <= E1; i += nwaves) {
    uint64_t word = 0;
    int before = 0;
    for (int g = 0; g < nruns; ++g) {
      const int eg = __builtin_amdgcn_readlane(rexp, g);
      before += eg < 64 * i;
      if ((eg >> 6) == i) word |= 1ull << (eg & 63);
    }
    const int x = lane + 64 * i;
    const int gx = x < E1 ? before + __popcll(word & below) : nruns;
    const int ox = lane_read(roff, gx & 63);
    if (x <= E1) o.expert_off[x] = gx < nruns ? ox : total;
  }
}

// The whole sort in one 1024-thread workgroup (S small). ids may live in LDS or global memory.
// When E1 * ceil(S / 64) words fit, every expert gets an S-bit set of its slots: the stable rank
// of slot f is the number of set bits below f (popcounts), and the count is the total — no ballot
// loop. Otherwise ranks come from wave ballots and per-wave counts.
inline __device__ void align_small_body(const int32_t* ids, int S, int E1, int bm, int cap,
                                        const AlignOut& o, AlignSmem& sm) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int words = (S + 63) >> 6;
  if (E1 * words <= kAlignBitmapWords) {
    for (int i = t; i < E1 * words; i += kAlignThreads) sm.bits[i] = 0ull;
    __syncthreads();
    for (int f = t; f < S; f += kAlignThreads) {
      int e = align_expert_of(ids, f, S, E1);
      if (e >= 0) atomicOr(&sm.bits[e * words + (f >> 6)], 1ull << (f & 63));
    }
    __syncthreads();
    // this thread's two experts (2t, 2t + 1) are counted straight into the layout's scan
    int c[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int e = 2 * t + h;
      if (e >= E1) continue;
      for (int w = 0; w < words; ++w) c[h] += __popcll(sm.bits[e * words + w]);
      sm.cnt[e] = c[h];
    }
    align_layout_core(c[0], c[1], sm.cnt, sm.off, E1, S, bm, cap, sm.s_wave, o, sm.tile_e, true);
    // off is complete (the layout's barriers); the scatter writes only valid-slot rows, which the
    // padding fill above never touches, so no barrier is needed between them
    for (int f = t; f < S; f += kAlignThreads) {
      int e = align_expert_of(ids, f, S, E1);
      if (e < 0) continue;
      const unsigned long long* b = sm.bits + e * words;
      int rank = __popcll(b[f >> 6] & ((1ull << (f & 63)) - 1ull));
      for (int w = 0; w < (f >> 6); ++w) rank += __popcll(b[w]);
      o.sorted_ids[sm.off[e] + rank] = f;
      if (o.sorted_w) o.sorted_w[sm.off[e] + rank] = o.topk_w[f];
    }
    return;
  }
  for (int e = t; e < E1; e += kAlignThreads) {
    sm.cnt[e] = 0;
    sm.run[e] = 0;
    for (int w = 0; w < kAlignWaves; ++w) sm.wcnt[w][e] = 0;
  }
  __syncthreads();
  for (int f = t; f < S; f += kAlignThreads) {
    int e = align_expert_of(ids, f, S, E1);
    if (e >= 0) atomicAdd(&sm.cnt[e], 1);
  }
  __syncthreads();
  align_layout_from_counts(sm.cnt, sm.off, E1, S, bm, cap, sm.s_wave, o, sm.tile_e);
  __syncthreads();
  for (int base = 0; base < S; base += kAlignThreads) {
    int f = base + t;
    int e = align_expert_of(ids, f, S, E1);
    uint64_t peers = match_peers(e, e >= 0);
    int rank = __popcll(peers & ((1ull << lane) - 1ull));
    if (e >= 0 && rank == 0) sm.wcnt[wave][e] = (uint16_t)__popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += sm.wcnt[w][e];
      const int pos = sm.off[e] + sm.run[e] + before + rank;
      o.sorted_ids[pos] = f;
      if (o.sorted_w) o.sorted_w[pos] = o.topk_w[f];
    }
    __syncthreads();
    for (int x = t; x < E1; x += kAlignThreads) {
      int s = 0;
      for (int w = 0; w < kAlignWaves; ++w) {
        s += sm.wcnt[w][x];
        sm.wcnt[w][x] = 0;
      }
      sm.run[x] += s;
    }
    __syncthreads();
  }
}

}  // namespace mxmoe
