// The whole MoE block for small batches in ONE launch: routing, the sorted layout, gate_up
// (SwiGLU, MXFP8 requantisation), down (weighted slot rows) and the fixed-order final sum.
//
// At decode sizes the block is a stream of expert weights (hundreds of MB at the 32-token and
// 128-token batches) and, between the launches of a multi-kernel block, the GPU does no streaming:
// each launch ramps up and drains, and routing, sorting and the final sum run with the HBM idle.
// "Ling-3.0-flash: Tối ưu hóa độ trễ giải mã lên 54% trên 4 GPU Blackwell" describes exactly this
// idle time between kernel nodes at batch 1 ("Hai loại thời gian nhàn rỗi") and the need for counts
// to stay on the GPU as indices ("Hình dạng của một bước batch-1"); "Tối ưu hiệu năng Kimi K3 trong
// vLLM" folds the top-k finalize into the GEMM epilogue to drop a launch and a round trip. Here
// every step is a role of one grid, and the roles overlap:
//
//   workgroups [0, R)        routers: route 4 tokens each (one per wave) and count themselves done.
//   next Q workgroups        quantisers: x -> MXFP8 codes and scales, counted when done.
//   next workgroup           layout: waits for the routers, builds the 16-row sorted layout
//                            (bit-identical to mxmoe_align) and publishes it with one agent-scope
//                            release.
//   next ng workgroups       gate_up units. When most experts are chosen, one per (routed expert,
//                            32-column intermediate chunk) plus the shared expert's (16-row group,
//                            chunk), issuing their first weight K-steps at once, before the
//                            layout tells them their rows; otherwise one per (chosen expert, chunk)
//                            once the layout names the chosen experts. They wait for the
//                            quantisers, multiply, and write their SwiGLU rows, requantised, at
//                            their sorted positions.
//   last nd workgroups       down units, one per (16-row layout tile, 64-column chunk): they wait
//                            for the layout, issue their weight K-steps, wait for their expert's
//                            gate_up count, then write weighted fp32 slot rows; the last unit to
//                            finish a (chunk, 8-token group) sums those tokens' slot rows in slot
//                            order and writes y.
//
// Every wait points to workgroups with lower ids (dispatched earlier), is bounded (after
// spin_limit polls it gives up, records a timeout and skips the dependent work, so every wave
// ends), and the status of the call is left in the control words for the host. Data crossing
// workgroups (which run on different XCDs, each with its own L2) is written and read with
// agent-scope coherent accesses (sc1), so no L2 write-back or invalidation is needed per unit;
// counters are agent-scope atomics. The control words live at the start of the workspace: they
// must be zero before the first call, and the last workgroup of every call resets them.
#include "align_dev.h"
#include "device.h"
#include "gemm_dev.h"
#include "kernels.h"
#include "route_dev.h"

namespace mxmoe {

namespace {

constexpr int kFThreads = 256;
constexpr int kFWaves = kFThreads / 64;
constexpr int kTokPerRouter = kFWaves;      // router workgroups route one token per wave
constexpr int kFinGroup = 16;               // tokens per final-sum group (one shared-expert tile)
constexpr int kCoherent = 16;               // cache policy sc1: agent-scope coherent access

enum : int {
  kCtlRouted = 0,   // router workgroups done
  kCtlReady = 1,    // layout published
  kCtlWgDone = 2,   // workgroups done
  kCtlTimeout = 3,  // a bounded wait gave up
  kCtlStatus = 4,   // result of the last call (not reset): 0 ok, 1 a wait gave up
  kCtlQuant = 5,    // quantiser workgroups done
  kCtlGuDone = 64,  // [E + 1] gate_up units done per expert
  kCtlFin = kCtlGuDone + kMaxExperts + 64,  // [DC * n_tg] final-sum arrivals
};
static_assert((kCtlFin + kFusedMaxFin) * 4 <= (int)kFusedCtlBytes, "control words");

struct FGrid {
  int R;                 // router workgroups [0, R)
  int q0, Q;             // quantiser workgroups [q0, q0 + Q); the layout workgroup is q0 + Q
  int g0, ng, d0, nd, total;
  int GC, DC;            // gate_up chunks (I / 32), down chunks (H / 64)
  int nks_g, nks_d;      // K-steps of gate_up (H / 128) and down (Ip / 128)
  int n_routed_units, n_units_g;
  int dcw;               // down workgroups per tile
  int n_tg;              // final-sum token groups
  int dense;             // most experts chosen: gate_up units per expert, weights issued first
  int expected_shared;   // gate_up units of the shared expert
};

__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait (wave-uniform) until *p >= target. Gives up after `limit` polls, recording a
// timeout, and returns false.
__device__ __forceinline__ bool wait_at_least(const int* p, int target, int limit, int* timeout) {
  for (int i = 0; i < limit; ++i) {
    if (__builtin_amdgcn_readfirstlane(ld_agent(p)) >= target) return true;
    __builtin_amdgcn_s_sleep(4);
  }
  if (lane_id() == 0) __hip_atomic_fetch_or(timeout, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return false;
}

struct LayoutSmem {
  unsigned long long bits[kFusedBitmapWords];
  int cnt[kMaxExperts + 1];
  int off[kMaxExperts + 2];
  int wsum[kFWaves], wtouch[kFWaves];
};
constexpr int kMaxSlotWords = kAlignSmallMaxSlots / 64;   // 64-slot words of the routing table
constexpr int kExpertWords = (kMaxExperts + 1 + 63) / 64;  // 64-expert words
struct UnitSmem {
  v4f part[kFWaves][4][64];               // split-K partial accumulators (one 16-row tile)
  unsigned long long slots[kFWaves][kMaxSlotWords];  // per wave: slots routed to its expert
  unsigned long long chosen[kFWaves][kExpertWords];  // per wave: experts anyone chose
  float shared[kFWaves][16][64 + 4];      // per wave: the shared expert's tile, for the final sum
};
union FusedSmem {
  LayoutSmem lay;
  UnitSmem u;
};

// ------------------------------------------------------------------------------ routers
__device__ __forceinline__ void role_route(const FusedArgs& a, const FGrid& gd, int r) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (a.logits_f32)
    route_tokens_any<true>(a.logits, r * kFWaves + wave, kFWaves * gd.R, a.T, a.E, a.top_k, lane,
                           a.ids, a.tw, nullptr);
  else
    route_tokens_any<false>(a.logits, r * kFWaves + wave, kFWaves * gd.R, a.T, a.E, a.top_k, lane,
                            a.ids, a.tw, nullptr);
  __syncthreads();  // every wave's ids and weights are stored (the barrier waits for them)
  if (threadIdx.x == 0)  // release: writes this XCD's L2 back before the count
    __hip_atomic_fetch_add(a.ctl + kCtlRouted, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------ layout
// The 16-row sorted layout of mxmoe_align from the routing ids, by one 256-thread workgroup:
// per-expert bitmaps of slots (a slot's stable rank is the number of set bits below it), a
// block scan of the padded counts, then every output written by consecutive threads.
__device__ __forceinline__ void role_layout(const FusedArgs& a, const FGrid& gd, LayoutSmem& sm) {
  constexpr int BM = 16;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int S = a.T * (a.top_k + 1), E1 = a.E + 1, words = (S + 63) >> 6;
  const AlignOut& o = a.lay;
  bool ok = true;
  if (wave == 0) ok = wait_at_least(a.ctl + kCtlRouted, gd.R, a.spin_limit, a.ctl + kCtlTimeout);
  if (t == 0) sm.wsum[0] = ok;
  __syncthreads();
  ok = sm.wsum[0] != 0;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // the routers' ids and weights
  for (int i = t; i < E1 * words; i += kFThreads) sm.bits[i] = 0ull;
  __syncthreads();
  for (int f = t; f < S && ok; f += kFThreads) {
    const int e = a.ids[f];
    if (e >= 0 && e < E1) atomicOr(&sm.bits[e * words + (f >> 6)], 1ull << (f & 63));
  }
  __syncthreads();
  for (int e = t; e < E1; e += kFThreads) {
    int c = 0;
    for (int w = 0; w < words; ++w) c += __popcll(sm.bits[e * words + w]);
    sm.cnt[e] = c;
  }
  __syncthreads();
  // thread t owns experts [t * ept, t * ept + ept): padded counts and touched flags, block scan
  const int ept = (E1 + kFThreads - 1) / kFThreads;
  int p = 0, nt = 0;
  for (int i = 0; i < ept; ++i) {
    const int e = t * ept + i;
    if (e < E1) {
      p += (sm.cnt[e] + BM - 1) / BM * BM;
      nt += sm.cnt[e] > 0;
    }
  }
  const int ip = wave_incl_scan(p), it = wave_incl_scan(nt);
  if (lane == 63) {
    sm.wsum[wave] = ip;
    sm.wtouch[wave] = it;
  }
  __syncthreads();
  int base = 0, tbase = 0, total = 0, ntouch = 0;
#pragma unroll
  for (int w = 0; w < kFWaves; ++w) {
    base += w < wave ? sm.wsum[w] : 0;
    tbase += w < wave ? sm.wtouch[w] : 0;
    total += sm.wsum[w];
    ntouch += sm.wtouch[w];
  }
  int ex = base + ip - p, tx = tbase + it - nt;
  for (int i = 0; i < ept; ++i) {
    const int e = t * ept + i;
    if (e >= E1) break;
    sm.off[e] = ex;
    if (sm.cnt[e] > 0) o.touched[tx++] = e;
    ex += (sm.cnt[e] + BM - 1) / BM * BM;
  }
  if (t == 0) {
    sm.off[E1] = total;
    *o.num_post_pad = total;
    *o.n_touched = ntouch;
  }
  __syncthreads();
  for (int e = t; e <= E1; e += kFThreads) o.expert_off[e] = sm.off[e];
  const int nb = a.cap / BM;
  for (int b = total / BM + t; b < nb; b += kFThreads) o.block_expert[b] = -1;
  for (int r = total + t; r < a.cap; r += kFThreads) {
    o.sorted_ids[r] = S;
    o.sorted_w[r] = 0.f;
  }
  for (int e = t; e < E1; e += kFThreads) {
    const int o0 = sm.off[e], o1 = sm.off[e + 1];
    for (int b = o0 / BM; b < o1 / BM; ++b) o.block_expert[b] = e;
    for (int r = o0 + sm.cnt[e]; r < o1; ++r) {
      o.sorted_ids[r] = S;
      o.sorted_w[r] = 0.f;
    }
  }
  for (int f = t; f < S && ok; f += kFThreads) {
    const int e = a.ids[f];
    if (e < 0 || e >= E1) continue;
    const unsigned long long* b = sm.bits + e * words;
    int rank = __popcll(b[f >> 6] & ((1ull << (f & 63)) - 1ull));
    for (int w = 0; w < (f >> 6); ++w) rank += __popcll(b[w]);
    o.sorted_ids[sm.off[e] + rank] = f;
    o.sorted_w[sm.off[e] + rank] = a.tw[f];
  }
  __syncthreads();
  if (t == 0 && !a.hold)  // release: the layout reaches memory before the flag
    __hip_atomic_store(a.ctl + kCtlReady, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------ quantisers
// x -> MXFP8 codes [T, H] and scale bytes [T, srs_H] (K-block order), four lanes per 32-element
// block as in the separate prologue (quant_dev.h), written through to the agent-coherent level
// for the gate_up units on other XCDs, which wait for the count of finished quantisers.
__device__ __forceinline__ void role_quant(const FusedArgs& a, int qwg) {
  const size_t gthr = (size_t)qwg * kFThreads + threadIdx.x;
  const size_t blk = gthr >> 2;
  const int part = (int)(gthr & 3), nbk = a.H / 32;
  if (blk < (size_t)a.T * nbk) {
    const size_t t = blk / nbk;
    const int kb = (int)(blk - t * nbk);
    const size_t off = t * a.H + (size_t)kb * 32 + 8 * part;
    const v4i q = *(const v4i*)(a.x + off);
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t u = (uint32_t)q[j];
      v[2 * j] = __uint_as_float(u << 16);
      v[2 * j + 1] = __uint_as_float(u & 0xFFFF0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    // the block's four lanes form a DPP quad: quad_perm [1,0,3,2], then [2,3,0,1]
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m), __float_as_int(m), 0xB1, 0xF, 0xF, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(m), __float_as_int(m), 0x4E, 0xF, 0xF, false)));
    const int se = mx_shared_exp<8>(m);
    const __amdgpu_buffer_rsrc_t rq = raw_rsrc(a.xq, (uint32_t)((size_t)a.T * a.H));
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(a.xs, (uint32_t)((size_t)a.T * a.srs_H));
    const v2i codes = v2i{(int)e4m3_quad(v[0], v[1], v[2], v[3], se),
                          (int)e4m3_quad(v[4], v[5], v[6], v[7], se)};
    __builtin_amdgcn_raw_buffer_store_b64(codes, rq, (uint32_t)off, 0, kCoherent);
    if (part == 0)
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(se + 127), rs,
                                           (uint32_t)(t * a.srs_H + kb), 0, kCoherent);
  }
  __syncthreads();  // every thread's codes have reached the coherent level
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(a.ctl + kCtlQuant, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------ gate_up
// Register ring depths (K-steps in flight per wave). gate_up: two, with the many concurrent units
// keeping the HBM queue full. down: three, the whole K of a 384-wide fp8 intermediate at once.
constexpr int kFRing = 2;
constexpr int kFDownRing = 3;

// Index of the r-th set bit of the wave's slot words (uniform, in LDS), or -1.
__device__ __forceinline__ int nth_slot(const unsigned long long* m, int words, int r) {
  for (int w = 0; w < words; ++w) {
    unsigned long long x = m[w];
    const int c = __popcll(x);
    if (r < c) {
      int pos = 0;
#pragma unroll
      for (int h = 32; h >= 1; h >>= 1) {
        const int lo = __popcll(x & ((1ull << h) - 1ull));
        if (r >= lo) {
          r -= lo;
          x >>= h;
          pos += h;
        }
      }
      return 64 * w + pos;
    }
    r -= c;
  }
  return -1;
}

// Weights of this wave's K-step i (global step kw + KS * i) into s; steps i >= nk (the padding
// of the ring's last group) read from an empty range, load nothing and multiply zeros, so the
// ring loop has no branch.
template <int WF>
__device__ __forceinline__ void issue_w(const GemmParams& p, const TileRows<1>& tr, int i, int nk,
                                        int kw, int KS, int lane, Stage<WF, 1>& s) {
  TileRows<1> t = tr;
  if (i >= nk) {
    t.w = raw_rsrc(nullptr, 0);
    t.ws = raw_rsrc(nullptr, 0);
  }
  load_b<WF, 1, 1, kNonTemporal>(p, t, i < nk ? kw + KS * i : 0, lane, s);
}

// MFMA A operand of step i: two 16-byte pieces of the row and its scale dword (agent-coherent:
// written by other workgroups of this launch); nothing for padding steps.
template <int WF>
__device__ __forceinline__ void issue_a(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t ras,
                                        uint32_t aoff, uint32_t asoff, int i, int nk, int kw,
                                        int KS, Stage<WF, 1>& s) {
  const int ks = i < nk ? kw + KS * i : 0;
  const uint32_t o = i < nk ? aoff : kOutOfRange, so = i < nk ? asoff : kOutOfRange;
  s.a[0][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, o, ks * KSTEP, kCoherent);
  s.a[0][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, o + 64u, ks * KSTEP, kCoherent);
  s.sa[0] = __builtin_amdgcn_raw_buffer_load_b32(ras, so, 4 * ks, kCoherent);
}

// The ring of D stages over this wave's nk K-steps (rounded up to whole groups), weights and A
// operands already issued for steps 0 .. D - 1.
template <int WF, int D, typename IssueW, typename IssueA>
__device__ __forceinline__ void ring_loop(Stage<WF, 1> (&buf)[D], int nk, int g, v4f (&acc)[1][4],
                                          IssueW&& iw, IssueA&& ia) {
  const int nkr = (nk + D - 1) / D * D;
  int k0 = 0;
  for (; k0 + D < nkr; k0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      mma_stage<WF, 1>(buf[s], 8 * g, acc);
      iw(k0 + s + D, buf[s]);
      ia(k0 + s + D, buf[s]);
    }
  }
#pragma unroll
  for (int s = 0; s < D; ++s) mma_stage<WF, 1>(buf[s], 8 * g, acc);
}

// Split-K: the unit's partial sums added in wave order into wave kw == 0's accumulators.
template <int KS>
__device__ __forceinline__ void reduce_split(UnitSmem& u, int wave, int kw, int lane, v4f (&acc)[1][4]) {
#pragma unroll
  for (int f = 0; f < 4; ++f) u.part[wave][f][lane] = acc[0][f];
  __syncthreads();
  if (kw == 0) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      v4f s = u.part[wave][f][lane];
#pragma unroll
      for (int w = 1; w < KS; ++w) {
        const v4f q = u.part[wave + w][f][lane];
        s[0] += q[0]; s[1] += q[1]; s[2] += q[2]; s[3] += q[3];
      }
      acc[0][f] = s;
    }
  }
  __syncthreads();
}

template <int WF, int KS>
__device__ __forceinline__ void role_gate_up(const FusedArgs& a, const FGrid& gd, int gwg, FusedSmem& sm) {
  constexpr int D = kFRing;
  constexpr int UPW = kFWaves / KS;
  UnitSmem& u = sm.u;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int unit = gwg * UPW + wave / KS, kw = wave % KS;
  if (unit >= gd.n_units_g) return;  // whole units only: a unit's waves skip together
  // Dense batches (most experts chosen): unit (expert e, chunk c), and the shared expert's 16-row
  // groups, with the first weight K-steps issued before the routing is known. Sparse batches: unit
  // (i-th chosen expert, chunk c), known once the routing is.
  int e = -1, c, grp = -1, i_chosen = 0;
  if (gd.dense) {
    if (unit < gd.n_routed_units) {
      e = unit / gd.GC;
      c = unit - e * gd.GC;
    } else {
      const int v = unit - gd.n_routed_units;
      grp = v / gd.GC;
      c = v - grp * gd.GC;
      e = a.E;
    }
  } else {
    i_chosen = unit / gd.GC;
    c = unit - i_chosen * gd.GC;
  }
  GemmParams p{};
  p.NKS = gd.nks_g;
  TileRows<1> tr;
  auto set_weights = [&](int ex) {
    constexpr int FB = Frag<WF>::bytes;
    const size_t wbytes = (size_t)(2 * a.I / 16) * gd.nks_g * FB;
    const size_t sbytes = (size_t)(2 * a.I / 64) * gd.nks_g * 256;
    tr.w = raw_rsrc(a.w13 + (size_t)ex * wbytes, (uint32_t)wbytes);
    tr.ws = raw_rsrc(a.s13 + (size_t)ex * sbytes, (uint32_t)sbytes);
    tr.nt0 = 4 * c;
  };
  const int nk = (gd.nks_g - kw + KS - 1) / KS;  // this wave's K-steps: kw, kw + KS, ...
  Stage<WF, 1> buf[D];
  auto issue_weights = [&]() {
#pragma unroll
    for (int s = 0; s < D; ++s) issue_w<WF>(p, tr, s, nk, kw, KS, lane, buf[s]);
  };
  if (gd.dense) {
    set_weights(e);
    issue_weights();
  }
  // the routing table (written by the router workgroups)
  if (!wait_at_least(a.ctl + kCtlRouted, gd.R, a.spin_limit, a.ctl + kCtlTimeout)) return;
  const int S = a.T * (a.top_k + 1), k1 = a.top_k + 1, words = (S + 63) >> 6;
  if (!gd.dense) {
    // the i-th smallest expert anyone chose
    const int ew = (a.E + 1 + 63) >> 6;
    for (int w = lane; w < ew; w += 64) u.chosen[wave][w] = 0ull;
    for (int f = lane; f < S; f += 64) {
      const int x = ld_agent(a.ids + f);
      if (x >= 0 && x <= a.E) atomicOr(&u.chosen[wave][x >> 6], 1ull << (x & 63));
    }
    int r = i_chosen;
    e = -1;
    for (int w = 0; w < ew && e < 0; ++w) {
      const unsigned long long m = u.chosen[wave][w];
      const int cnt = __popcll(m);
      if (r < cnt) {
        unsigned long long x = m;
        int pos = 0;
        for (int h = 32; h >= 1; h >>= 1) {
          const int lo = __popcll(x & ((1ull << h) - 1ull));
          if (r >= lo) { r -= lo; x >>= h; pos += h; }
        }
        e = 64 * w + pos;
      }
      r -= cnt;
    }
    e = __builtin_amdgcn_readfirstlane(e);
    if (e < 0) return;
    set_weights(e);
    issue_weights();
  }
  // this expert's slots, in flat order (= token order)
  int ne = 0;
  if (grp < 0) {
    for (int w = 0; w < words; ++w) {
      const int f = 64 * w + lane;
      const unsigned long long m = __ballot(f < S && ld_agent(a.ids + f) == e);
      if (lane == 0) u.slots[wave][w] = m;
      ne += __popcll(m);
    }
  } else {
    ne = min(16, a.T - 16 * grp);
  }
  if (ne <= 0) return;  // an expert nobody chose (its prefetched weights are dropped)
  const bool xready = wait_at_least(a.ctl + kCtlQuant, gd.Q, a.spin_limit, a.ctl + kCtlTimeout);
  const __amdgpu_buffer_rsrc_t rx = raw_rsrc(a.xq, (uint32_t)((size_t)a.T * a.H));
  const __amdgpu_buffer_rsrc_t rxs = raw_rsrc(a.xs, (uint32_t)((size_t)a.T * a.srs_H));
  const __amdgpu_buffer_rsrc_t rh = raw_rsrc(a.h, (uint32_t)((size_t)a.cap * a.h_stride));
  const __amdgpu_buffer_rsrc_t rhs = raw_rsrc(a.hs, (uint32_t)((size_t)a.cap * a.srs_I));
  int off_e = -1;  // the expert's first sorted row, read from the layout at the first epilogue
  const int passes = (ne + 15) / 16;
  for (int pass = 0; pass < passes; ++pass) {
    const int r0 = 16 * pass;  // first rank of this pass
    int tok;
    if (grp >= 0) tok = 16 * grp + n < a.T ? 16 * grp + n : -1;
    else {
      const int f = r0 + n < ne ? nth_slot(u.slots[wave], words, r0 + n) : -1;
      tok = f >= 0 ? f / k1 : -1;
    }
    const uint32_t xoff = xready && tok >= 0 ? (uint32_t)tok * (uint32_t)a.H + 16u * g : kOutOfRange;
    const uint32_t xsoff = xready && tok >= 0 ? (uint32_t)tok * (uint32_t)a.srs_H : kOutOfRange;
    if (pass > 0) issue_weights();  // a later 16-row tile streams the slice again
#pragma unroll
    for (int s = 0; s < D; ++s) issue_a<WF>(rx, rxs, xoff, xsoff, s, nk, kw, KS, buf[s]);
    v4f acc[1][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[0][f] = v4f{0.f, 0.f, 0.f, 0.f};
    ring_loop<WF, D>(buf, nk, g, acc,
                     [&](int i, Stage<WF, 1>& st) { issue_w<WF>(p, tr, i, nk, kw, KS, lane, st); },
                     [&](int i, Stage<WF, 1>& st) { issue_a<WF>(rx, rxs, xoff, xsoff, i, nk, kw, KS, st); });
    if constexpr (KS > 1) {
      reduce_split<KS>(u, wave, kw, lane, acc);
      if (kw != 0) continue;  // the epilogue is wave 0's; every wave stays for the next pass
    }
    // Epilogue: SwiGLU and MXFP8 requantisation along I; the rows go to their sorted positions
    // (the layout's offset of the expert plus the row's rank), written through to the agent-
    // coherent level for the down units on other XCDs.
    if (off_e < 0) {
      const bool ready = wait_at_least(a.ctl + kCtlReady, 1, a.spin_limit, a.ctl + kCtlTimeout);
      off_e = ready ? __builtin_amdgcn_readfirstlane(ld_agent(a.lay.expert_off + e)) : a.cap;
    }
    const int ic0 = 32 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a0 = silu(acc[0][0][i]) * acc[0][1][i];
      const float a1 = silu(acc[0][2][i]) * acc[0][3][i];
      const float m = row16_max(fmaxf(fabsf(a0), fabsf(a1)));
      const int se = mx_shared_exp<8>(m);
      const uint32_t c2 = e4m3_pair(a0, a1, se);
      const int rank = (grp >= 0 ? 16 * grp : 0) + r0 + 4 * g + i;
      if (rank < (grp >= 0 ? a.T : ne)) {
        const uint32_t row = (uint32_t)(off_e + rank);
        const uint32_t ho = row * (uint32_t)a.h_stride + (uint32_t)ic0;
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)c2, rh, ho + n, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(c2 >> 8), rh, ho + 16 + n, 0, kCoherent);
        if (n == 0)
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(se + 127), rhs,
                                               row * (uint32_t)a.srs_I + c, 0, kCoherent);
        // K padding of the intermediate (I not a multiple of 128): zero codes, finite scales
        if (a.Ip > a.I && 32 * (c + 1) == a.I) {
          for (int col = a.I + n; col < a.Ip; col += 16)
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)0, rh, row * (uint32_t)a.h_stride + col,
                                                 0, kCoherent);
          if (n == 0)
            for (int kb = a.I / 32; kb < a.Ip / 32; ++kb)
              __builtin_amdgcn_raw_buffer_store_b8((uint8_t)127, rhs,
                                                   row * (uint32_t)a.srs_I + kb, 0, kCoherent);
        }
      }
    }
  }
  if (kw != 0) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the rows have reached the coherent level
  if (lane == 0)
    __hip_atomic_fetch_add(a.ctl + kCtlGuDone + e, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------ down
// Down units: (16-row layout tile, 64-column chunk). A routed expert's tile writes its weighted
// fp32 slot rows and then counts them per (chunk, 16-token group). The shared expert's tiles come
// last in the layout (and in the grid): every token has exactly one shared slot, in token order,
// so shared tile g holds tokens 16 g .. 16 g + 15; it waits until all routed slot rows of those
// tokens are counted and writes y = sum over the slots in slot order (routed slots 0 .. top_k - 1,
// then its own, the shared slot top_k: the order of the separate final-sum kernel).
template <int WF, int KS>
__device__ __forceinline__ void role_down(const FusedArgs& a, const FGrid& gd, int dwg, FusedSmem& sm) {
  constexpr int D = kFDownRing;
  UnitSmem& u = sm.u;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  int b, c, kw;
  if (KS == 1) {
    b = dwg / gd.dcw;
    c = (dwg - b * gd.dcw) * kFWaves + wave;
    kw = 0;
  } else {
    b = dwg / gd.DC;
    c = dwg - b * gd.DC;
    kw = wave;
  }
  const int S = a.T * (a.top_k + 1), k1 = a.top_k + 1;
  bool work = c < gd.DC;
  // the layout (wave-uniform decisions; a split-K unit's waves decide alike)
  if (work) work = wait_at_least(a.ctl + kCtlReady, 1, a.spin_limit, a.ctl + kCtlTimeout);
  int e = -1;
  if (work) {
    work = 16 * b < __builtin_amdgcn_readfirstlane(ld_agent(a.lay.num_post_pad));
    if (work) e = __builtin_amdgcn_readfirstlane(ld_agent(a.lay.block_expert + b));
    work = work && e >= 0 && e <= a.E;
  }
  if (KS > 1) {  // a unit's waves must agree before the reduction barrier
    if (wave == 0 && lane == 0) u.part[0][0][0][0] = work ? 1.f : 0.f;
    __syncthreads();
    work = u.part[0][0][0][0] != 0.f;
    __syncthreads();
  }
  if (!work) return;
  // the tile's rows before any weight load: lane n's A row and the epilogue rows 4g + i
  const int r0 = 16 * b;
  const int sid_n = ld_agent(a.lay.sorted_ids + r0 + n);
  int rsid[4];
  float rw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rsid[i] = ld_agent(a.lay.sorted_ids + r0 + 4 * g + i);
    rw[i] = ld_agent(a.lay.sorted_w + r0 + 4 * g + i);
  }
  GemmParams p{};
  p.NKS = gd.nks_d;
  TileRows<1> tr;
  {
    constexpr int FB = Frag<WF>::bytes;
    const size_t wbytes = (size_t)(a.H / 16) * gd.nks_d * FB;
    const size_t sbytes = (size_t)(a.H / 64) * gd.nks_d * 256;
    tr.w = raw_rsrc(a.w2 + (size_t)e * wbytes, (uint32_t)wbytes);
    tr.ws = raw_rsrc(a.s2 + (size_t)e * sbytes, (uint32_t)sbytes);
    tr.nt0 = 4 * c;
  }
  const int nk = (gd.nks_d - kw + KS - 1) / KS;
  Stage<WF, 1> buf[D];
#pragma unroll
  for (int s = 0; s < D; ++s) issue_w<WF>(p, tr, s, nk, kw, KS, lane, buf[s]);
  const int need = e == a.E ? gd.expected_shared : gd.GC;
  const bool ready = wait_at_least(a.ctl + kCtlGuDone + e, need, a.spin_limit, a.ctl + kCtlTimeout);
  const __amdgpu_buffer_rsrc_t rh = raw_rsrc(a.h, (uint32_t)((size_t)a.cap * a.h_stride));
  const __amdgpu_buffer_rsrc_t rhs = raw_rsrc(a.hs, (uint32_t)((size_t)a.cap * a.srs_I));
  const bool row_ok = ready && sid_n < S;
  const uint32_t aoff = row_ok ? (uint32_t)(r0 + n) * (uint32_t)a.h_stride + 16u * g : kOutOfRange;
  const uint32_t asoff = row_ok ? (uint32_t)(r0 + n) * (uint32_t)a.srs_I : kOutOfRange;
#pragma unroll
  for (int s = 0; s < D; ++s) issue_a<WF>(rh, rhs, aoff, asoff, s, nk, kw, KS, buf[s]);
  v4f acc[1][4];
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[0][f] = v4f{0.f, 0.f, 0.f, 0.f};
  ring_loop<WF, D>(buf, nk, g, acc,
                   [&](int i, Stage<WF, 1>& st) { issue_w<WF>(p, tr, i, nk, kw, KS, lane, st); },
                   [&](int i, Stage<WF, 1>& st) { issue_a<WF>(rh, rhs, aoff, asoff, i, nk, kw, KS, st); });
  if constexpr (KS > 1) {
    reduce_split<KS>(u, wave, kw, lane, acc);
    if (kw != 0) return;
  }
  const __amdgpu_buffer_rsrc_t ro = raw_rsrc(a.slots, (uint32_t)((size_t)S * a.H * 4));
  if (e != a.E) {
    // routed: weighted fp32 slot rows, written through, then counted per 16-token group
    if (ready) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (rsid[i] >= S) continue;
        // four adjacent columns per lane (the prepack's W2 row order), one coherent 16-byte store
        __builtin_amdgcn_raw_buffer_store_b128(
            v4i{__float_as_int(rw[i] * acc[0][0][i]), __float_as_int(rw[i] * acc[0][1][i]),
                __float_as_int(rw[i] * acc[0][2][i]), __float_as_int(rw[i] * acc[0][3][i])},
            ro, (uint32_t)(((size_t)rsid[i] * a.H + 64 * c + 4 * n) * 4), 0, kCoherent);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const int mytg = (lane < 16 && sid_n < S) ? (sid_n / k1) / kFinGroup : -1;
    unsigned long long todo = __ballot(mytg >= 0);
    while (todo) {  // rows are in token order: a few runs of equal groups
      const int leader = __ffsll(todo) - 1;
      const int cur = __shfl(mytg, leader);
      const unsigned long long same = __ballot(mytg == cur);
      if (lane == 0)
        __hip_atomic_fetch_add(a.ctl + kCtlFin + c * gd.n_tg + cur, (int)__popcll(same),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      todo &= ~same;
    }
    return;
  }
  // shared expert: this tile's rows are tokens t0 .. t0 + 15 (slot top_k of each), weight 1
  const int t0 = (ld_agent(a.lay.sorted_ids + r0) / k1) & ~(kFinGroup - 1);
  const int tg = t0 / kFinGroup, ntok = min(kFinGroup, a.T - t0);
  // stage its own contribution, row-major [token][column], for the row-major final sum
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 4; ++f) u.shared[wave][4 * g + i][4 * n + f] = rw[i] * acc[0][f][i];
  const bool all_in = wait_at_least(a.ctl + kCtlFin + c * gd.n_tg + tg, ntok * a.top_k,
                                    a.spin_limit, a.ctl + kCtlTimeout);
  // lane l: token t0 + l / 4, columns 16 (l % 4) .. + 16 of this chunk
  const int tr_ = lane >> 2, q = lane & 3, t = t0 + tr_;
  const int col = 64 * c + 16 * q;
  float acc16[16];
#pragma unroll
  for (int x = 0; x < 16; ++x) acc16[x] = 0.f;
  if (all_in && t < a.T) {
    for (int j0 = 0; j0 < a.top_k; j0 += 4) {
      v4i v[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int jj = min(j0 + j, a.top_k - 1);
        const uint32_t o = (uint32_t)((((size_t)t * k1 + jj) * a.H + col) * 4);
#pragma unroll
        for (int x = 0; x < 4; ++x)
          v[j][x] = __builtin_amdgcn_raw_buffer_load_b128(ro, o + 16u * x, 0, kCoherent);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j0 + j < a.top_k)
#pragma unroll
          for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) acc16[4 * x + y] += __int_as_float(v[j][x][y]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  if (t < a.T) {
    uint32_t o[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const float s0 = acc16[2 * x] + u.shared[wave][tr_][16 * q + 2 * x];
      const float s1 = acc16[2 * x + 1] + u.shared[wave][tr_][16 * q + 2 * x + 1];
      o[x] = bf16_pair(s0, s1);
    }
    uint16_t* yr = a.y + (size_t)t * a.H + col;
    *(v4i*)yr = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    *(v4i*)(yr + 8) = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
  }
}

// ------------------------------------------------------------------------------ kernel
// The last workgroup to finish resets the control words for the next call and leaves the status.
__device__ __forceinline__ void finish_workgroup(const FusedArgs& a, const FGrid& gd) {
  __shared__ int last;
  __syncthreads();  // every wave of this workgroup is done (its stores have completed)
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(a.ctl + kCtlWgDone, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) == gd.total - 1;
  __syncthreads();
  if (!last) return;
  for (int i = threadIdx.x; i <= a.E; i += kFThreads) a.ctl[kCtlGuDone + i] = 0;
  for (int i = threadIdx.x; i < gd.DC * gd.n_tg; i += kFThreads) a.ctl[kCtlFin + i] = 0;
  if (threadIdx.x == 0) {
    a.ctl[kCtlStatus] = ld_agent(a.ctl + kCtlTimeout) ? 1 : 0;
    a.ctl[kCtlTimeout] = 0;
    a.ctl[kCtlRouted] = 0;
    a.ctl[kCtlReady] = 0;
    a.ctl[kCtlWgDone] = 0;
  }
}

template <int WF, int KS>
__global__ __launch_bounds__(kFThreads) void k_fused(FusedArgs a, FGrid gd) {
  __shared__ FusedSmem sm;
  const int wg = blockIdx.x;
  if (wg < gd.R) role_route(a, gd, wg);
  else if (wg < gd.q0 + gd.Q) role_quant(a, wg - gd.q0);
  else if (wg == gd.q0 + gd.Q) role_layout(a, gd, sm.lay);
  else if (wg < gd.d0) role_gate_up<WF, KS>(a, gd, wg - gd.g0, sm);
  else role_down<WF, KS>(a, gd, wg - gd.d0, sm);
  finish_workgroup(a, gd);
}

// Split K over a unit's four waves when few units would carry the whole weight stream (a
// handful of tokens): each wave then has a quarter of the K-steps in flight.
constexpr int kFusedSplitMaxUnits = 1024;

}  // namespace

bool fused_fits(int wf, int T, int H, int E, int top_k, int I) {
  if (wf == WF_BF16 || a_is_fp4(wf) || T < 1) return false;
  const int S = T * (top_k + 1);
  if (T > kFusedMaxT || S > kAlignSmallMaxSlots) return false;
  if ((E + 1) * ((S + 63) / 64) > kFusedBitmapWords) return false;
  if ((H / 64) * ((T + kFinGroup - 1) / kFinGroup) > kFusedMaxFin) return false;
  return true;
}

hipError_t launch_fused(int wf, const FusedArgs& a, hipStream_t st) {
  FGrid gd{};
  const int S = a.T * (a.top_k + 1);
  gd.R = (a.T + kTokPerRouter - 1) / kTokPerRouter;
  gd.GC = a.I / 32;
  gd.DC = a.H / 64;
  gd.nks_g = a.H / KSTEP;
  gd.nks_d = a.Ip / KSTEP;
  const int active = (a.E < S - a.T ? a.E : S - a.T) + 1;  // experts that can hold rows
  const bool split = (active * gd.GC <= kFusedSplitMaxUnits) &&
                     (active * gd.DC <= kFusedSplitMaxUnits);
  const int KS = split ? 4 : 1;
  gd.dense = S - a.T >= a.E;  // at least as many routed slots as experts
  const int tiles_shared = (a.T + 15) / 16;  // the shared expert's 16-row groups
  if (gd.dense) {
    gd.n_routed_units = a.E * gd.GC;
    gd.n_units_g = gd.n_routed_units + tiles_shared * gd.GC;
    gd.expected_shared = tiles_shared * gd.GC;
  } else {
    gd.n_routed_units = 0;
    gd.n_units_g = (S < a.E + 1 ? S : a.E + 1) * gd.GC;  // the chosen experts (at most S of them)
    gd.expected_shared = gd.GC;
  }
  const int upw = kFWaves / KS;
  gd.ng = (gd.n_units_g + upw - 1) / upw;
  gd.dcw = (gd.DC + kFWaves - 1) / kFWaves;
  const int tiles = a.cap / 16;
  gd.nd = KS == 1 ? tiles * gd.dcw : tiles * gd.DC;
  gd.q0 = gd.R;
  gd.Q = (int)(((size_t)a.T * (a.H / 32) * 4 + kFThreads - 1) / kFThreads);
  gd.g0 = gd.q0 + gd.Q + 1;
  gd.d0 = gd.g0 + gd.ng;
  gd.total = gd.d0 + gd.nd;
  gd.n_tg = (a.T + kFinGroup - 1) / kFinGroup;
  const dim3 grid(gd.total), block(kFThreads);
#define MXMOE_FUSED(W, K) hipLaunchKernelGGL((k_fused<W, K>), grid, block, 0, st, a, gd)
  if (wf == WF_FP8) {
    if (KS == 4) MXMOE_FUSED(WF_FP8, 4);
    else MXMOE_FUSED(WF_FP8, 1);
  } else {
    if (KS == 4) MXMOE_FUSED(WF_FP4, 4);
    else MXMOE_FUSED(WF_FP4, 1);
  }
#undef MXMOE_FUSED
  return hipGetLastError();
}

}  // namespace mxmoe
