// Grouped GEMMs of the MoE block on gfx950 block-scaled MFMA.
//
//   gate_up: for every slot row r of expert e, [gate | up](r) = x^(token(r)) . W13_e^T, then
//            SwiGLU a = SiLU(gate) * up in the epilogue and requantisation of a to MXFP8 along I
//            (bf16 rounding for bf16 weights).
//   down   : d(r) = a^(r) . W2_e^T, then the top-k weighted combine w(r) * d(r) back to the token
//            (written per slot for a fixed-order sum, or accumulated with fp32 atomics).
// The routed and the shared expert go through the same pass: the shared expert is just another
// entry of the routing table ("Lần theo điểm nghẽn: Tối ưu MiniMax M3 trên AMD Instinct MI355X",
// shared-expert passage, Fig. 4). Fusing the combine into the down epilogue follows the deferred
// top-k finalize of "Tối ưu hiệu năng Kimi K3 trong vLLM" (one launch and one intermediate
// write/read fewer).
//
// Small-M launcher (decode): one wave per (column chunk, tile); D K-steps of operands are in flight
// per wave (a register ring), since at decode M the weights are read once and HBM latency is the
// limit. Units are ordered so that the tiles of one expert on one column chunk are consecutive on
// the same XCD (workgroups go round-robin over the 8 XCDs, each with its own L2): an expert with
// more than one tile reads its weights from HBM once, the grouped-MoE program ordering of the
// MiniMax-M3 page's local-shapes passage.
#include <algorithm>
#include <atomic>

#include "device.h"
#include "gemm_dev.h"
#include "kernels.h"

namespace mxmoe {

namespace {

// acc[mt][f][i] is C[row 4g+i of tile mt][column n of fragment f]. Fragments 0/1 are gate/up of
// intermediate columns chunk*32 + 0..15, fragments 2/3 of chunk*32 + 16..31. hrow[mt][i]: the
// intermediate row that row 4g+i of tile mt is stored to (its layout row, or its slot in the
// slot-order plan), -1 for none.
template <int WF, int MT>
__device__ __forceinline__ void epilogue_gate_up(const GemmParams& p, const v4f (&acc)[MT][4],
                                                 const int (&hrow)[MT][4], int chunk, int n) {
  const int ic0 = 32 * chunk;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = hrow[mt][i];
      float a0 = silu(acc[mt][0][i]) * acc[mt][1][i];
      float a1 = silu(acc[mt][2][i]) * acc[mt][3][i];
      if (a_is_fp4(WF)) {  // E2M1 intermediate: 16 bytes per 32 columns, two codes per byte
        const float m = row16_max(fmaxf(fabsf(a0), fabsf(a1)));
        const int se = mx_shared_exp<2>(m);
        const uint32_t b2 = e2m1_pack_pair(a0, a1, se);
        if (rr >= 0) {
          uint8_t* hr = p.h + (size_t)rr * p.h_stride + ic0 / 2;
          if (!(n & 1)) {
            hr[n / 2] = (uint8_t)b2;
            hr[8 + n / 2] = (uint8_t)(b2 >> 8);
          }
          if (n == 0) p.hs[(size_t)rr * p.h_srs + chunk] = (uint8_t)(se + 127);
        }
      } else if (WF != WF_BF16) {
        const float m = row16_max(fmaxf(fabsf(a0), fabsf(a1)));
        int se = mx_shared_exp<8>(m);
        if (rr >= 0) {
          uint8_t* hr = p.h + (size_t)rr * p.h_stride + ic0;
          const uint32_t c2 = e4m3_pair(a0, a1, se);
          hr[n] = (uint8_t)c2;
          hr[16 + n] = (uint8_t)(c2 >> 8);
          if (n == 0) p.hs[(size_t)rr * p.h_srs + chunk] = (uint8_t)(se + 127);
        }
      } else if (rr >= 0) {
        uint16_t* hr = (uint16_t*)(p.h + (size_t)rr * p.h_stride) + ic0;
        hr[n] = (uint16_t)f32_to_bf16_bits(a0);
        hr[16 + n] = (uint16_t)f32_to_bf16_bits(a1);
      }
    }
  }
  // K padding of the intermediate (I not a multiple of 128): zero codes, finite scales.
  if (p.Ip > p.I && 32 * (chunk + 1) == p.I) {
    for (int mt = 0; mt < MT; ++mt)
      for (int i = 0; i < 4; ++i) {
        const int rr = hrow[mt][i];
        if (rr < 0) continue;
        if (WF != WF_BF16) {
          const int cb = a_is_fp4(WF) ? 2 : 1;  // codes per byte
          for (int c = p.I / cb + n; c < p.Ip / cb; c += 16) p.h[(size_t)rr * p.h_stride + c] = 0;
          if (n == 0)
            for (int kb = p.I / 32; kb < p.Ip / 32; ++kb)
              p.hs[(size_t)rr * p.h_srs + kb] = 127;
        } else {
          uint16_t* hr = (uint16_t*)(p.h + (size_t)rr * p.h_stride);
          for (int c = p.I + n; c < p.Ip; c += 16) hr[c] = 0;
        }
      }
  }
}

// Destination rows of the sorted layout: row 4g+i of tile mt is layout row m0 + 16 mt + 4g + i.
template <int MT>
__device__ __forceinline__ void layout_rows(int m0, int r1, int g, int (&hrow)[MT][4]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = m0 + 16 * mt + 4 * g + i;
      hrow[mt][i] = rr < r1 ? rr : -1;
    }
}

// Output columns of a down fragment: the prepack interleaves the rows of W2 so that fragment f
// of a wave's 64-column chunk gives lane n column 4n + f, i.e. each lane holds four adjacent
// output columns of its rows and stores them as one 8-byte (bf16) or 16-byte (fp32) piece.
__device__ __forceinline__ void store_down_row(const GemmParams& p, int sid, float wt, float v0,
                                               float v1, float v2, float v3, int c0) {
  if (p.combine == 3) {
    uint2 o;
    o.x = bf16_pair(wt * v0, wt * v1);
    o.y = bf16_pair(wt * v2, wt * v3);
    *(uint2*)((uint16_t*)p.out32 + (size_t)sid * p.H + c0) = o;
  } else if (p.combine == 1) {
    *(v4f*)(p.out32 + (size_t)sid * p.H + c0) = v4f{wt * v0, wt * v1, wt * v2, wt * v3};
  } else {
    float* orow = p.out32 + (size_t)(sid / p.k1) * p.H + c0;
    atomicAdd(orow, wt * v0);
    atomicAdd(orow + 1, wt * v1);
    atomicAdd(orow + 2, wt * v2);
    atomicAdd(orow + 3, wt * v3);
  }
}

// combine 1: fp32 slot rows [S, H]; 2: fp32 atomics into token rows [T, H]; 3: bf16 slot rows.
template <int MT>
__device__ __forceinline__ void epilogue_down(const GemmParams& p, const v4f (&acc)[MT][4], int m0,
                                              int r1, int chunk, int n, int g) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = m0 + 16 * mt + 4 * g + i;
      if (rr >= r1) continue;
      const int sid = p.sorted_ids[rr];
      if (sid >= p.S) continue;
      store_down_row(p, sid, p.sorted_w[rr], acc[mt][0][i], acc[mt][1][i], acc[mt][2][i],
                     acc[mt][3][i], 64 * chunk + 4 * n);
    }
  }
}

// Down epilogue of the small-M launcher (one 16-row tile, rows 4g + i of the lane): slot id and
// routing weight of each row were loaded when the wave started.
__device__ __forceinline__ void epilogue_down_rows(const GemmParams& p, const v4f (&acc)[4],
                                                   const int (&rsid)[4], const float (&rw)[4],
                                                   int chunk, int n) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (rsid[i] >= p.S) continue;
    store_down_row(p, rsid[i], rw[i], acc[0][i], acc[1][i], acc[2][i], acc[3][i],
                   64 * chunk + 4 * n);
  }
}

// Fused final rounding (atomic combine, small-M launcher): every wave that did a tile of column
// chunk `chunk` bumps that chunk's counter once its atomics are acknowledged; the wave that
// completes the count (one per tile with work) rounds the chunk's 64 columns of all T token rows
// to bf16, reading the sums with agent-scope loads (the level the atomics are performed at). No
// agent-scope fence is used: on this GPU it writes back and invalidates the whole L2 of the XCD,
// which every wave of the pass would pay.
__device__ __forceinline__ void finalize_chunk_if_last(const GemmParams& p, int chunk, int lane) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int last = 0;
  if (lane == 0)
    last = __hip_atomic_fetch_add(p.chunk_done + chunk, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT) == *p.num_post_pad / p.block_m - 1;
  last = __builtin_amdgcn_readfirstlane(last);
  if (!last) return;
  const int col = 64 * chunk + 4 * (lane & 15);
  for (int t = lane >> 4; t < p.T; t += 4) {
    float* src = p.out32 + (size_t)t * p.H + col;
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      v[c] = __hip_atomic_load(src + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint2 o;
    o.x = bf16_pair(v[0], v[1]);
    o.y = bf16_pair(v[2], v[3]);
    *(uint2*)(p.y + (size_t)t * p.H + col) = o;
  }
}

// ------------------------------------------------------------------------------ small-M
// Slot-order plan: the rows of expert slot es (slot ids in slot order) into rows[], returning
// their count. A routed expert scans the routing ids, 64 slots per ballot with 16 loads in
// flight; a token chooses an expert at most once, so it has at most T rows (the host keeps
// T <= kSlotOrderMaxT). Shared tile j holds the shared slots (slot k of each token) of tokens
// 16j .. 16j + 15. The order is the sorted layout's (stable by slot), so a tile holds the same
// rows there and here. Every lane of the wave takes part; the count is wave-uniform.
__device__ __forceinline__ int so_rows(const GemmParams& p, int es, int lane, int* rows) {
  if (es >= p.E) {
    const int t0 = 16 * (es - p.E);
    const int nr = p.T - t0 < 16 ? p.T - t0 : 16;
    if (lane < nr) rows[lane] = (t0 + lane) * p.k1 + (p.k1 - 1);
    return nr;
  }
  int cnt = 0;
  for (int c0 = 0; c0 < p.S; c0 += 64 * 16) {
    int v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int s = c0 + 64 * j + lane;
      v[j] = s < p.S ? p.topk_ids[s] : -1;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool m = v[j] == es;
      const uint64_t b = __builtin_amdgcn_ballot_w64(m);
      const int idx = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                (uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
      if (m && idx < kSlotOrderMaxT) rows[idx] = c0 + 64 * j + lane;
      cnt += __builtin_popcountll(b);
    }
  }
  return cnt < kSlotOrderMaxT ? cnt : kSlotOrderMaxT;
}

// Slot-order plan, gate_up units of column chunk 0: the expert slot's rows (slot ids, p.S past the
// count) and, once per expert, its count, for the down pass. Same wave as so_rows.
__device__ __forceinline__ void so_record(const GemmParams& p, int es, int nr, int lane,
                                          const int* rows) {
  if (es < p.E) {
    int32_t* l = p.so_list + (size_t)es * p.so_cap;
    for (int i = lane; i < p.so_cap; i += 64) l[i] = i < nr ? rows[i] : p.S;
    if (lane == 0) p.so_cnt[es] = nr;
  } else {
    const int t0 = 16 * (es - p.E);
    if (lane < nr) p.so_list[(size_t)p.E * p.so_cap + t0 + lane] = rows[lane];
    if (lane == 0 && t0 == 0) p.so_cnt[p.E] = p.T;
  }
}

// KS > 1 (few units, 16-row blocks): KS waves share a unit, wave w taking K-steps w, w + KS, ...;
// their accumulators are added in LDS in wave order (a fixed order) and wave 0 runs the epilogue.
// With a few hundred single-wave units (a handful of tokens) each wave's K stream is a chain of
// memory round trips; split over KS waves the chain is KS times shorter.
// SO: the slot-order plan (one wave per unit, one 16-row tile at a time).
// The MFMAs of one K-step with the activation fragments of stage sa_src and the weight fragments
// of stage sb_src (the second chunk of a paired unit).
template <int WF, int MT>
__device__ __forceinline__ void mma_stage_b(const Stage<WF, MT>& sa_src, const Stage<WF, MT>& sb_src,
                                            int ash, v4f (&acc)[MT][4]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    v8i a8;
    a8.lo = sa_src.a[mt][0];
    a8.hi = a_is_fp4(WF) ? v4i{0, 0, 0, 0} : sa_src.a[mt][1];
    mma_frags<WF>(a8, (int)(sa_src.sa[mt] >> ash), sb_src.b, (int)sb_src.sb, acc[mt]);
  }
}

// NG: 4-fragment weight groups per unit (2: a unit covers two adjacent column chunks with one
// activation stream; slot-order gate_up with fp4 weights, where a chunk's K-step is 4 KB).
template <int WF, int MT, bool GATE_UP, int D, int KS, int AUX = 0, bool SO = false, int NG = 1>
__global__ __launch_bounds__(64 * KS) void k_gemm_stream(GemmParams p, int n_chunks, int n_blocks) {
  static_assert(NG == 1 || (GATE_UP && SO), "paired chunks: slot-order gate_up only");
  static_assert(GATE_UP || MT == 1, "the down epilogue of this launcher handles one 16-row tile");
  static_assert(KS == 1 || MT == 1, "split K reduces one 16-row tile");
  static_assert(!SO || (KS == 1 && MT == 1), "slot order: one wave, one 16-row tile");
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int wave = KS > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  // Unit order: XCD x = blockIdx % 8 takes the x-th contiguous range of the units that have rows
  // (the grid is sized for the layout's capacity; ranges cut from the real tile count give every
  // XCD the same work, measured 57.9 -> 55.6 us for the 32-token gate_up); units run chunk-major,
  // tiles fastest, so the tiles of one expert on one chunk share an XCD.
  const int nb = SO ? p.E + p.so_tiles : (p.cap_units ? n_blocks : *p.num_post_pad / p.block_m);
  const int total = n_chunks * nb;
  const int per_xcd = (total + 7) >> 3;
  const bool ranges = p.xcd_order && !p.cap_units;
  if (ranges && (int)(blockIdx.x >> 3) >= per_xcd) return;
  const int u = ranges ? (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3) : (int)blockIdx.x;
  if (u >= total) return;
  const int chunk = u / nb, blk = u - chunk * nb;
  // slot order: rows r0 .. r1 - 1 of the unit are so_r[r] (slot ids)
  __shared__ int so_r[SO ? kSlotOrderMaxT : 1];
  int r0, r1, e;
  TileRows<MT> tr;
  // Register ring of D stages; the host picks D dividing NKS, so the steady-state loop issues
  // the loads of group k0 + D while multiplying group k0 without any branch, and the last group
  // is peeled. Weight loads of the first group go out before the (dependent) row lookup.
  Stage<WF, MT> buf[D];
  Stage<WF, MT> bufB[NG == 2 ? D : 1];  // second chunk's weights (its activation part is unused)
  TileRows<MT> trB;
  if constexpr (SO) {
    // the unit's expert is known: its first weight K-steps go out before the scan for its rows
    // (an expert without rows then drops D K-steps of one chunk)
    e = blk < p.E ? blk : p.E;
    tile_weights<WF, MT>(p, e, chunk * 4 * NG, tr);
    trB = tr;
    trB.nt0 = tr.nt0 + 4;
#pragma unroll
    for (int s = 0; s < D; ++s) {
      load_b<WF, MT, MT, AUX>(p, tr, s, lane, buf[s]);
      if constexpr (NG == 2) load_b<WF, MT, MT, AUX>(p, trB, s, lane, bufB[s]);
    }
    r0 = 0;
    r1 = so_rows(p, blk, lane, so_r);
    if (GATE_UP && chunk == 0) so_record(p, blk, r1, lane, so_r);
    if (r1 == 0) {  // wave-uniform
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      return;
    }
  } else {
    r0 = blk * p.block_m;
    e = p.block_expert[blk];
    if (e < 0) return;  // a tile past the layout's last (units over the capacity)
    r1 = r0 + p.block_m;
    tile_weights<WF, MT>(p, e, chunk * 4, tr);
  }
  // slot id of unit row r (p.S: none)
  auto row_slot = [&](int r) -> int {
    if constexpr (SO) return r < r1 ? so_r[r] : p.S;
    else return r < r1 ? p.sorted_ids[r] : p.S;
  };
  // slot order: intermediate row of unit row r (the expert's rows, then the shared tile's offset)
  const int hbase = SO ? e * p.so_cap + (blk < p.E ? 0 : 16 * (blk - p.E)) : 0;
  for (int m0 = r0; m0 < r1; m0 += 16 * MT) {
    v4f acc[MT][4], accB[NG == 2 ? MT : 1][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (NG == 2) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int f = 0; f < 4; ++f) accB[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    const int nk = p.NKS / KS;  // K-steps of this wave: global step wave + KS * i
    if (!SO || m0 != r0) {  // slot order: the first tile's ring went out before the scan
#pragma unroll
      for (int s = 0; s < D; ++s) {
        load_b<WF, MT, MT, AUX>(p, tr, wave + KS * s, lane, buf[s]);
        if constexpr (NG == 2) load_b<WF, MT, MT, AUX>(p, trB, wave + KS * s, lane, bufB[s]);
      }
    }
    // down: slot id and routing weight of the lane's four output rows, fetched now so the
    // epilogue does not wait for them
    int rsid[4];
    float rw[4];
    if (!GATE_UP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rsid[i] = row_slot(m0 + 4 * g + i);
        if constexpr (SO) rw[i] = rsid[i] < p.S ? p.topk_w[rsid[i]] : 0.0f;
        else rw[i] = p.sorted_w[m0 + 4 * g + i];
      }
    }
    if constexpr (SO) {  // gate_up: token row of the slot; down: the expert's intermediate row
      const int sid = row_slot(m0 + n);
      const int ar = GATE_UP ? sid / p.k1 : hbase + m0 + n;
      tr.aoff[0] = sid < p.S ? (uint32_t)ar * (uint32_t)p.a_stride + 16u * g : kOutOfRange;
      tr.asoff[0] = sid < p.S ? (uint32_t)ar * (uint32_t)p.a_srs : kOutOfRange;
    } else {
      tile_act_rows<WF, MT, GATE_UP>(p, m0, r1, n, g, tr);
    }
#pragma unroll
    for (int s = 0; s < D; ++s) load_a<WF, MT>(tr, wave + KS * s, buf[s]);
    int k0 = 0;
    for (; k0 + D < nk; k0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        mma_stage<WF, MT>(buf[s], 8 * g, acc);
        if constexpr (NG == 2) {
          mma_stage_b<WF, MT>(buf[s], bufB[s], 8 * g, accB);
          load_b<WF, MT, MT, AUX>(p, trB, wave + KS * (k0 + s + D), lane, bufB[s]);
        }
        load_stage<WF, MT, AUX>(p, tr, wave + KS * (k0 + s + D), lane, buf[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) {
      mma_stage<WF, MT>(buf[s], 8 * g, acc);
      if constexpr (NG == 2) mma_stage_b<WF, MT>(buf[s], bufB[s], 8 * g, accB);
    }
    if constexpr (KS > 1) {
      __shared__ v4f part[KS][4][64];
#pragma unroll
      for (int f = 0; f < 4; ++f) part[wave][f][lane] = acc[0][f];
      __syncthreads();
      if (wave != 0) return;  // one 16-row tile per unit (block_m 16): nothing left for the others
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        v4f t = part[0][f][lane];
#pragma unroll
        for (int w = 1; w < KS; ++w) {
          const v4f q = part[w][f][lane];
          t[0] += q[0]; t[1] += q[1]; t[2] += q[2]; t[3] += q[3];
        }
        acc[0][f] = t;
      }
    }
    if constexpr (GATE_UP) {
      int hrow[MT][4];
      if constexpr (SO) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = m0 + 4 * g + i;
          hrow[0][i] = r < r1 ? hbase + r : -1;
        }
      } else {
        layout_rows<MT>(m0, r1, g, hrow);
      }
      epilogue_gate_up<WF, MT>(p, acc, hrow, chunk * NG, n);
      if constexpr (NG == 2) epilogue_gate_up<WF, MT>(p, accB, hrow, chunk * 2 + 1, n);
    } else {
      epilogue_down_rows(p, acc[0], rsid, rw, chunk, n);
    }
  }
  if (!SO && !GATE_UP && p.y) finalize_chunk_if_last(p, chunk, lane);
}

// Small-M down pass with the 16-row activation tile shared by a workgroup: its 4 waves take 4
// consecutive 64-column chunks of one tile of the sorted layout (slot order: of one expert slot,
// its tiles in turn), and the tile's intermediate rows (16 rows of Ip codes and their scale bytes,
// contiguous in the layout, gathered by slot in slot order) are copied into LDS once
// instead of being gathered by every wave at every K-step; each wave then streams its own weight
// slice through the same register ring as k_gemm_stream, and the sums are the same (same K order
// per wave, no split). At decode the activation loads were a third of the down pass's vector-memory
// instructions: a timing variant without them ran the 32-token down pass in 25.9 against 28.7 us
// and the 128-token MXFP4 one in 34.1 against 39.2 us. Dynamic LDS: rows at pitch a_stride + 16
// (the 16 rows of one MFMA operand read then start in different banks), then the scale rows.
constexpr int kSaWaves = 4;
constexpr int kSaMaxLds = 48 * 1024;

__host__ __device__ inline int sa_pitch(int a_stride) { return a_stride + 16; }
__host__ __device__ inline int sa_lds_bytes(int a_stride, int a_srs) {
  return 16 * sa_pitch(a_stride) + 16 * a_srs;
}

template <int WF, int D, int AUX, bool SO = false>
__global__ __launch_bounds__(64 * kSaWaves) void k_gemm_down_sa(GemmParams p, int n_groups,
                                                                 int n_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sa_lds[];
  constexpr bool A4 = a_is_fp4(WF);
  constexpr int SB = A4 ? KSTEP / 2 : KSTEP;  // code bytes of a row per K-step
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // unit (chunk group, tile), chunk-group-major, in contiguous per-XCD ranges (as k_gemm_stream)
  const int nb = SO ? p.E + p.so_tiles : (p.cap_units ? n_blocks : *p.num_post_pad / 16);
  const int total = n_groups * nb;
  const int per_xcd = (total + 7) >> 3;
  const bool ranges = p.xcd_order && !p.cap_units;
  if (ranges && (int)(blockIdx.x >> 3) >= per_xcd) return;
  const int u = ranges ? (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3) : (int)blockIdx.x;
  if (u >= total) return;  // uniform over the workgroup
  const int grp = u / nb, blk = u - grp * nb;
  const int chunk = grp * kSaWaves + wave;
  // Rows: sorted layout, the 16-row tile r0 of the layout; slot order, the expert slot's
  // intermediate rows hbase, hbase + 1, ... (its count from gate_up, or the shared tile's tokens),
  // the first tile copied before the count is known (rows past it are never stored).
  int e, r0, cnt, hbase, t0 = 0;
  if constexpr (SO) {
    e = blk < p.E ? blk : p.E;
    if (blk < p.E) {
      cnt = p.so_cnt[e];
      hbase = e * p.so_cap;
    } else {
      t0 = 16 * (blk - p.E);
      cnt = p.T - t0 < 16 ? p.T - t0 : 16;
      hbase = p.E * p.so_cap + t0;
    }
    r0 = 0;
  } else {
    r0 = blk * 16;
    cnt = 16;
    hbase = 0;
    e = p.block_expert[blk];
    if (e < 0) return;  // a tile past the layout's last (uniform over the workgroup)
  }
  TileRows<1> tr;
  tile_weights<WF, 1>(p, e, chunk * 4, tr);
  const int pitch = sa_pitch(p.a_stride);
  const int cbytes = 16 * p.a_stride, sbytes = 16 * p.a_srs;
  const __amdgpu_buffer_rsrc_t ra = raw_rsrc(p.a, p.a_bytes);
  const __amdgpu_buffer_rsrc_t ras = raw_rsrc(p.as, p.as_bytes);
  const uint8_t* arow = sa_lds + n * pitch;
  const uint32_t* srow = (const uint32_t*)(sa_lds + 16 * pitch + n * p.a_srs);
  // The first tile's row copy goes out before the count is read. Its weights go out with it when
  // few experts lack rows (so_spec), else one K-step before the count and the rest after: an
  // expert without rows then reads one step of its slice, not all of it (at three K-steps a
  // unit's ring is its whole weight slice). Measured down pass: 32 tokens over 128 experts (13%
  // without rows) 30.1 us all weights first, 28.6 us all after, 28.0 us one step first; 128
  // tokens MXFP4 35.0 us all first against 36.6 us all after.
  const bool spec = !SO || p.so_spec;
  for (int m0 = 0;; m0 += 16) {
    Stage<WF, 1> buf[D];
    if (spec || m0 > 0) {
#pragma unroll
      for (int s = 0; s < D; ++s) load_b<WF, 1, 1, AUX>(p, tr, s, lane, buf[s]);
    } else {
      load_b<WF, 1, 1, AUX>(p, tr, 0, lane, buf[0]);  // one K-step before the count
    }
    // slot of each of the lane's four output rows (p.S: none)
    int rsid[4];
    float rw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m0 + 4 * g + i;
      if constexpr (SO) {
        if (blk < p.E) rsid[i] = p.so_list[hbase + (r < p.so_cap ? r : 0)];
        else rsid[i] = t0 + r < p.T ? (t0 + r) * p.k1 + (p.k1 - 1) : p.S;
      } else {
        rsid[i] = p.sorted_ids[r0 + r];
        rw[i] = p.sorted_w[r0 + r];
      }
    }
    // The tile's rows and scale rows into LDS (16 consecutive rows), in 16-byte pieces, every load
    // of a batch issued before the first LDS store.
    const uint32_t a0 = (uint32_t)(r0 + hbase + m0) * (uint32_t)p.a_stride;
    const uint32_t s0 = (uint32_t)(r0 + hbase + m0) * (uint32_t)p.a_srs;
    constexpr int kB = 4;
    for (int base = 16 * threadIdx.x; base < cbytes + sbytes; base += 16 * 64 * kSaWaves * kB) {
      v4i v[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int o = base + 16 * 64 * kSaWaves * j;
        v[j] = o < cbytes ? __builtin_amdgcn_raw_buffer_load_b128(ra, a0 + o, 0, 0)
                          : __builtin_amdgcn_raw_buffer_load_b128(ras, o < cbytes + sbytes ? s0 + (o - cbytes) : kOutOfRange, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int o = base + 16 * 64 * kSaWaves * j;
        if (o < cbytes) {
          const int row = o / p.a_stride, col = o - row * p.a_stride;
          *(v4i*)(sa_lds + row * pitch + col) = v[j];
        } else if (o < cbytes + sbytes) {
          *(v4i*)(sa_lds + 16 * pitch + (o - cbytes)) = v[j];
        }
      }
    }
    if constexpr (SO) {
      if (m0 == 0) {
        if (cnt == 0) {  // an expert without rows (uniform over the workgroup)
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          return;
        }
        if (!spec) {
#pragma unroll
          for (int s = 1; s < D; ++s) load_b<WF, 1, 1, AUX>(p, tr, s, lane, buf[s]);
        }
      }
    }
    __syncthreads();
    if constexpr (SO) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (m0 + 4 * g + i >= cnt) rsid[i] = p.S;  // list entries past the count
        rw[i] = rsid[i] < p.S ? p.topk_w[rsid[i]] : 0.0f;
      }
    }
    v4f acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
    auto mma_step = [&](int ks, const Stage<WF, 1>& st) {
      v8i a8;
      a8.lo = *(const v4i*)(arow + ks * SB + 16 * g);
      a8.hi = A4 ? v4i{0, 0, 0, 0} : *(const v4i*)(arow + ks * SB + 64 + 16 * g);
      const uint32_t sa = srow[ks];
      mma_frags<WF>(a8, (int)(sa >> (8 * g)), st.b, (int)st.sb, acc);
    };
    const int nk = p.NKS;
    int k0 = 0;
    for (; k0 + D < nk; k0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        mma_step(k0 + s, buf[s]);
        load_b<WF, 1, 1, AUX>(p, tr, k0 + s + D, lane, buf[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) mma_step(k0 + s, buf[s]);
    epilogue_down_rows(p, acc, rsid, rw, chunk, n);
    if (m0 + 16 >= cnt) break;
    __syncthreads();  // every wave's reads of this tile come before the next tile's copy
  }
  if (!SO && p.y) finalize_chunk_if_last(p, chunk, lane);
}

// ------------------------------------------------------------------------------ large-M
// Prefill launcher: a workgroup of 4 waves computes a 128-row x 256-column tile (rows of one expert
// from the sorted layout); each wave owns 64 columns (4 weight fragments) for all 128 rows, i.e.
// 8 x 4 block-scaled MFMAs per 128-K step, with the 128 fp32 accumulators in AGPRs.
//
// The gathered 128 x 128-byte activation tile of a K-step (and its scale dwords) is shared by the
// 4 waves, so it travels global -> LDS by the buffer unit's direct LDS loads, double-buffered. The
// weight fragments are private to a wave and go straight into registers (two slots, one K-step
// ahead): staging them through LDS too doubled the LDS traffic and tripled the stage size. A
// direct LDS load writes lane i's bytes at (base + size * i), so the global address each lane
// requests decides the LDS layout: activation rows are 128 bytes with the eight 16-byte units of
// row r stored at unit c ^ (r & 7) — the 16 rows an MFMA operand read touches then spread over all
// banks (measured on gfx950: ~198 B/clk/CU for this read pattern, against ~119 with 16-byte row
// padding). Stages are 17 KB and the kernel stays within 256 registers, so two workgroups share a
// CU and each one's load waits are covered by the other's MFMAs (measured on the 8K-token
// prefill: gate_up 274 us, down 253 us, against 316 / 312 us for one workgroup per CU with every
// operand staged through a three-deep LDS ring).
// With E2M1 activations a row of the K-step is 64 bytes (four 16-byte units, one K-block each),
// stored at pitch 64 with unit c of row r at c ^ a4_swz(r): reading 16 rows at one K-block then
// takes each 16-byte slot of a 128-byte (and of a 256-byte) bank window once.
// Stage completion is a wait on the wave's own load counter followed by a workgroup barrier,
// written as one asm statement (the compiler's barrier would also wait for loads it cannot see).
constexpr int kTileM = 128;
constexpr int kTileWaves = 4;
constexpr int kLdsPitch = KSTEP;

// Unit swizzle of an E2M1 activation row in LDS (r & 15 = the row within its 16-row group).
__device__ __forceinline__ int a4_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }


// Wait until at most N of this wave's vector-memory loads are outstanding and its LDS reads are
// done, then barrier.
template <int N>
__device__ __forceinline__ void wait_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// gate_up epilogue of a 128-row x 256-column tile: the workgroup's 4 waves hold the gate/up
// pairs of 4 consecutive MX blocks (128 intermediate columns) of every row. SwiGLU and the MXFP8
// requantisation run in registers; codes and scale bytes are staged in LDS, then each row's 128
// code bytes go out as 16-byte stores (8 lanes per row) and its 4 scale bytes as one dword (the
// scale layout is in K-block order). Rows of padding slots are written too (their codes are zero
// since their activation rows read as zero), so the down pass can read every row of a tile.
// With E2M1 intermediates (a_is_fp4) a row of the tile is 64 code bytes, two codes per byte.
template <int WF, int LDS_BYTES>
__device__ __forceinline__ void epilogue_gate_up_tile(const GemmParams& p, const v4f (&acc)[8][4],
                                                      int r0, int chunk, int wave, int n, int g,
                                                      int tid, uint8_t* lds, int mtv) {
  constexpr bool A4 = a_is_fp4(WF);
  constexpr int kRowBytes = A4 ? 64 : 128;   // code bytes of a row of the tile
  constexpr int kPitch = kRowBytes + 16;     // code row pitch in LDS
  static_assert(kTileM * kPitch + kTileM * 4 <= LDS_BYTES, "gate_up staging exceeds the LDS buffer");
  uint8_t* codes = lds;                      // [128][kPitch]
  uint32_t* scales = (uint32_t*)(lds + kTileM * kPitch);  // [128] dwords, byte = wave
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt >= mtv) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * g + i;
      const float a0 = silu(acc[mt][0][i]) * acc[mt][1][i];
      const float a1 = silu(acc[mt][2][i]) * acc[mt][3][i];
      const float m = row16_max(fmaxf(fabsf(a0), fabsf(a1)));
      if constexpr (A4) {
        const int se = mx_shared_exp<2>(m);
        const uint32_t b2 = e2m1_pack_pair(a0, a1, se);
        if (!(n & 1)) {
          codes[row * kPitch + 16 * wave + n / 2] = (uint8_t)b2;
          codes[row * kPitch + 16 * wave + 8 + n / 2] = (uint8_t)(b2 >> 8);
        }
        if (n == 0) ((uint8_t*)scales)[4 * row + wave] = (uint8_t)(se + 127);
      } else {
        const int se = mx_shared_exp<8>(m);
        const uint32_t c2 = e4m3_pair(a0, a1, se);
        codes[row * kPitch + 32 * wave + n] = (uint8_t)c2;
        codes[row * kPitch + 32 * wave + 16 + n] = (uint8_t)(c2 >> 8);
        if (n == 0) ((uint8_t*)scales)[4 * row + wave] = (uint8_t)(se + 127);
      }
    }
  }
  __syncthreads();
  constexpr int kUnits = kRowBytes / 16;     // 16-byte stores per row
#pragma unroll
  for (int j = 0; j < kTileM * kUnits / 256; ++j) {
    const int c = tid + 256 * j, row = c / kUnits, unit = c % kUnits;
    if (row < 16 * mtv)
      *(v4i*)(p.h + (size_t)(r0 + row) * p.h_stride + kRowBytes * chunk + 16 * unit) =
          *(const v4i*)(codes + row * kPitch + 16 * unit);
  }
  if (tid < 16 * mtv)
    *(uint32_t*)(p.hs + (size_t)(r0 + tid) * p.h_srs + 4 * chunk) = scales[tid];
}

// Barrier for LDS reuse only: waits for this wave's LDS operations, then for the workgroup. The
// release fence of __syncthreads also waits for every global store the wave has outstanding,
// which put the write latency of each staged pass of the down epilogue on the critical path.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// down epilogue with bf16 slot rows, straight from registers: each lane holds four adjacent
// columns (4n .. 4n + 3 of the wave's 64) of rows 16 mt + 4g + i and writes them as one 8-byte
// store, so the 16 lanes of a row cover its 128-byte segment in one store instruction; rows of
// padding slots are skipped. (With the earlier column order, four columns 16 apart per lane, the
// tile went through an LDS staging pass instead; direct 8-byte stores measured the same at 8K
// tokens and 89 -> 82 us at 4096 tokens x 512 experts.) Slot ids and weights of the tile's rows
// are in LDS (row_sid, row_w).
__device__ __forceinline__ void epilogue_down_tile(const GemmParams& p, const v4f (&acc)[8][4],
                                                   int wchunk, int n, int g, const int* row_sid,
                                                   const float* row_w, int mtv) {
  uint16_t* out16 = (uint16_t*)p.out32;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    if (mt >= mtv) break;
    const v4f wt = *(const v4f*)(row_w + 16 * mt + 4 * g);
    const v4i sd = *(const v4i*)(row_sid + 16 * mt + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint2 o;
      o.x = bf16_pair(wt[i] * acc[mt][0][i], wt[i] * acc[mt][1][i]);
      o.y = bf16_pair(wt[i] * acc[mt][2][i], wt[i] * acc[mt][3][i]);
      if (sd[i] < p.S) *(uint2*)(out16 + (size_t)sd[i] * p.H + 64 * wchunk + 4 * n) = o;
    }
  }
}

// Slots (rows with slot id < S) among the 128 rows of a tile; they precede the tile's padding.
// Every lane of the wave takes part; the count is returned to all of them.
__device__ __forceinline__ int tile_slots(const int32_t* rows, int S, int lane) {
  const uint64_t lo = __builtin_amdgcn_ballot_w64(rows[lane] < S);
  const uint64_t hi = __builtin_amdgcn_ballot_w64(rows[64 + lane] < S);
  return __builtin_popcountll(lo) + __builtin_popcountll(hi);
}

// LDS stage of the large-M launcher: the 128 x 128-byte activation tile and its scale dwords
// (per wave 256 bytes; waves 2 and 3 fill an unused slot, see below).
struct TileLds {
  static constexpr int a = 0;
  static constexpr int as = kTileM * kLdsPitch;
  static constexpr int bytes = as + kTileWaves * 256;
};

template <int WF, bool GATE_UP, bool PIPE, bool PRIO = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_tile(GemmParams p, int n_chunks, int n_blocks, int sub_shift) {
  using L = TileLds;
  constexpr int MT = kTileM / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * L::bytes];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int total = n_chunks * n_blocks;
  // Unit order. Units are tile-major (the column chunks of a 128-row tile adjacent: the gathered
  // activation tile is fetched once and reused from L2). Workgroups go round-robin over the 8
  // XCDs (XCD x = blockIdx % 8 runs positions blockIdx / 8), each with its own L2; every XCD
  // takes runs of xcd_run consecutive units in turn. The launcher sets runs of 4 tiles: a run
  // shares its activation tiles and its experts' weight slices in one L2, and every XCD works
  // through the whole expert list, popular experts and one-tile experts alike. Measured against
  // one contiguous range per XCD and against plain linear order (run 1): 8K tokens x 128
  // experts gate_up 208 against 226 and 239 us; 4K tokens x 512 experts gate_up 112-115 against
  // 182 and 117 us, down 93-95 against ~100 us (chunk-major ranges). The grid is a whole number of
  // 8 * xcd_run workgroups, so the mapping covers every unit.
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3, run = p.xcd_run;
  const int u = (pos / run) * (8 * run) + xcd * run + pos % run;
  if (u >= total) return;
  const int blk = u / n_chunks;
  const int chunk = u - blk * n_chunks;
  // n_blocks counts 128-row tiles; a layout block of 256 rows (sub_shift 1) holds two of them
  const int r0 = blk * kTileM;
  if (r0 >= *p.num_post_pad) return;
  // A tile holds rows of one expert, its slots first and then padding. 16-row groups of padding
  // only (mt >= mtv) skip their MFMAs and their epilogue; down skips the same groups, so the
  // intermediate rows gate_up leaves unwritten there are never used. Under skewed routing many
  // experts fill a fraction of a tile (4096 tokens x 512 experts: a quarter of the tiles hold
  // fewer than 16 slots).
  // Not in the fp8 down pass (three or four K-steps at these shapes): there the count's load at
  // the start of every tile cost more than the skipped MFMAs saved (8K-token down 210 -> 216 us).
  constexpr bool kSkip = GATE_UP || WF != WF_FP8;
  const int mtv = kSkip ? __builtin_amdgcn_readfirstlane(
                              (tile_slots(p.sorted_ids + r0, p.S, lane) + 15) >> 4)
                        : kTileM / 16;
  if (mtv == 0) return;  // a padding-only half of a 256-row layout block
  const int e = p.block_expert[blk >> sub_shift];
  const int wchunk = chunk * kTileWaves + wave;
  TileRows<1> tr;
  tile_weights<WF, 1>(p, e, wchunk * 4, tr);
  __shared__ __attribute__((aligned(16))) int row_sid[kTileM];
  __shared__ __attribute__((aligned(16))) float row_w[kTileM];
  if (!GATE_UP && tid < kTileM) {
    row_sid[tid] = p.sorted_ids[r0 + tid];
    row_w[tid] = p.sorted_w[r0 + tid];
  }
  const v4i ra = rsrc_words(p.a, p.a_bytes);
  const v4i ras = rsrc_words(p.as, p.as_bytes);
  auto act_row = [&](int r, uint32_t stride) -> uint32_t {
    if (r >= r0 + 16 * mtv) return kOutOfRange;
    if (GATE_UP) {
      const int sid = p.sorted_ids[r];
      return sid < p.S ? (uint32_t)(sid / p.k1) * stride : kOutOfRange;
    }
    return (uint32_t)r * stride;
  };
  // Per wave and K-step, 32 activation rows: E4M3 rows of 128 bytes in 4 loads of 8 rows, E2M1
  // rows of 64 bytes in 2 loads of 16 rows (lane: row lane / 4, unit lane % 4).
  constexpr bool A4 = a_is_fp4(WF);
  constexpr int kAPitch = A4 ? KSTEP / 2 : kLdsPitch;  // LDS (and global per-step) row bytes
  constexpr int kALoads = A4 ? 2 : 4;
  constexpr int kARows = 32 / kALoads;                 // rows per load
  uint32_t aoff[kALoads];
#pragma unroll
  for (int j = 0; j < kALoads; ++j) {
    if constexpr (A4) {
      const int lr = lane >> 2;
      aoff[j] = act_row(r0 + 32 * wave + kARows * j + lr, (uint32_t)p.a_stride) +
                16u * ((lane & 3) ^ a4_swz(lr));
    } else {
      aoff[j] = act_row(r0 + 32 * wave + kARows * j + (lane >> 3), (uint32_t)p.a_stride) +
                16u * ((lane & 7) ^ (lane >> 3));
    }
  }
  const uint32_t asoff = wave < 2 ? act_row(r0 + 64 * wave + lane, (uint32_t)p.a_srs) : kOutOfRange;
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)lds;
  auto issue_a = [&](int stage, int ks, uint32_t oob) {
    const uint32_t st = lds0 + stage * L::bytes;
#pragma unroll
    for (int j = 0; j < kALoads; ++j)
      lds_load16(ra, st + L::a + (32 * wave + kARows * j) * kAPitch, aoff[j] | oob, ks * kAPitch);
    lds_load4(ras, st + L::as + 256 * wave, asoff | oob, 4 * ks);
  };
  v4f acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};
  const int u0 = A4 ? (g ^ a4_swz(n)) << 4 : (g ^ (n & 7)) << 4;
  const int u1 = ((4 + g) ^ (n & 7)) << 4;
  Stage<WF, 1> bs[2];
  // The lane's A fragment of 16-row group mt: two 16-byte units (E4M3) or one (E2M1, the upper
  // half of the operand is zero) and the row's scale dword.
  auto a_frag = [&](int stage, int mt, v8i& a8, uint32_t& sa) {
    const uint8_t* st = lds + stage * L::bytes;
    const uint8_t* base = st + L::a + n * kAPitch;
    a8.lo = *(const v4i*)(base + mt * 16 * kAPitch + u0);
    a8.hi = A4 ? v4i{0, 0, 0, 0} : *(const v4i*)(base + mt * 16 * kAPitch + u1);
    sa = *(const uint32_t*)(st + L::as + 4 * (16 * mt + n));
  };
  // MV (compile time): the 16-row groups the loop multiplies, mtv rounded up to 1, 2, 4 or 8.
  auto compute = [&](int stage, const Stage<WF, 1>& b, int mt0, int mt1, auto MVC) {
    constexpr int MV = decltype(MVC)::value;
#pragma unroll
    for (int mt = mt0; mt < (mt1 < MV ? mt1 : MV); ++mt) {
      v8i a8;
      uint32_t sa;
      a_frag(stage, mt, a8, sa);
      mma_frags<WF>(a8, (int)(sa >> (8 * g)), b.b, (int)b.sb, acc[mt]);
    }
  };
  const int nks = p.NKS;
  load_b<WF, 1, 1>(p, tr, 0, lane, bs[0]);
  issue_a(0, 0, 0u);
  wait_loads_barrier<0>();
  // Step ks multiplies stage / weight slot ks % 2. The loads of step ks + 1 go out while it runs:
  // the activation tile (no registers) after the first two 16-row groups, the weights after the
  // fourth (at 255 registers; issued after the second, both weight slots would be live across
  // more MFMAs and the fp8 kernel spills). By then the compiler has waited for this step's
  // weights, so its count of outstanding loads cannot make it wait for the new ones (the
  // activation loads are invisible to it). The
  // loop runs over pairs of steps so that the register slots are compile-time; after an odd step
  // count the last step runs alone (its loads were issued by the step before it).
  // PIPE: the next step's weights go out first, so they have a whole step to arrive, and the
  // activation fragments are read one 16-row group ahead of their MFMAs (two register sets).
  // PRIO: the wave's priority is raised while it issues the step's MFMAs.
  auto step_pipe = [&](auto SLOT, int ks, auto MVC) {
    constexpr int s = decltype(SLOT)::value;
    constexpr int MV = decltype(MVC)::value;
    const uint32_t oob = ks + 1 < nks ? 0u : kOutOfRange;
    TileRows<1> tn = tr;
    if (oob) tn.w = raw_rsrc(p.w, 0);
    load_b<WF, 1, 1>(p, tn, ks + 1 < nks ? ks + 1 : 0, lane, bs[1 - s]);
    __builtin_amdgcn_sched_barrier(0);
    v8i a8[2];
    uint32_t sa[2];
    a_frag(s, 0, a8[0], sa[0]);
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    static_for<MT>([&](auto MTI) {
      constexpr int mt = decltype(MTI)::value;
      if constexpr (mt + 1 < MT) a_frag(s, mt + 1, a8[(mt + 1) & 1], sa[(mt + 1) & 1]);
      if constexpr (mt == 1) issue_a(1 - s, ks + 1, oob);
      if constexpr (mt < MV)
        mma_frags<WF>(a8[mt & 1], (int)(sa[mt & 1] >> (8 * g)), bs[s].b, (int)bs[s].sb, acc[mt]);
      __builtin_amdgcn_sched_barrier(0);
    });
    if (PRIO) __builtin_amdgcn_s_setprio(0);
    wait_loads_barrier<0>();
  };
  auto step = [&](auto SLOT, int ks, auto MVC) {
    if constexpr (PIPE) {
      step_pipe(SLOT, ks, MVC);
      return;
    }
    constexpr int s = decltype(SLOT)::value;
    const uint32_t oob = ks + 1 < nks ? 0u : kOutOfRange;
    compute(s, bs[s], 0, 2, MVC);
    __builtin_amdgcn_sched_barrier(0);
    issue_a(1 - s, ks + 1, oob);
    __builtin_amdgcn_sched_barrier(0);
    compute(s, bs[s], 2, 4, MVC);
    __builtin_amdgcn_sched_barrier(0);
    TileRows<1> tn = tr;
    if (oob) tn.w = raw_rsrc(p.w, 0);
    load_b<WF, 1, 1>(p, tn, ks + 1 < nks ? ks + 1 : 0, lane, bs[1 - s]);
    __builtin_amdgcn_sched_barrier(0);
    compute(s, bs[s], 4, MT, MVC);
    __builtin_amdgcn_sched_barrier(0);
    wait_loads_barrier<0>();
  };
  auto k_loop = [&](auto MVC) {
    int ks = 0;
    for (; ks + 1 < nks; ks += 2) {
      step(std::integral_constant<int, 0>{}, ks, MVC);
      step(std::integral_constant<int, 1>{}, ks + 1, MVC);
    }
    if (ks < nks) {  // odd step count: the last step alone (nothing to load)
      compute(0, bs[0], 0, MT, MVC);
      // every wave's reads of stage 0 are done before the gate_up epilogue stages codes there
      if constexpr (GATE_UP) lds_barrier();
    }
  };
  // One copy of the loop per group count, so that every loop's MFMAs are unconditional. With
  // E4M3 activations the kernel is at the register limit, and more than two copies spill.
  if constexpr (a_is_fp4(WF) || WF == WF_FP4) {
    if (mtv > 4) k_loop(std::integral_constant<int, 8>{});
    else if (mtv > 2) k_loop(std::integral_constant<int, 4>{});
    else if (mtv > 1) k_loop(std::integral_constant<int, 2>{});
    else k_loop(std::integral_constant<int, 1>{});
  } else if constexpr (kSkip) {
    if (mtv > 2) k_loop(std::integral_constant<int, 8>{});
    else k_loop(std::integral_constant<int, 2>{});
  } else {
    k_loop(std::integral_constant<int, 8>{});
  }
  if constexpr (GATE_UP) {
    epilogue_gate_up_tile<WF, sizeof(lds)>(p, acc, r0, chunk, wave, n, g, tid, lds, mtv);
  } else {
    if (p.combine == 3)
      epilogue_down_tile(p, acc, wchunk, n, g, row_sid, row_w, mtv);
    else epilogue_down<MT>(p, acc, r0, r0 + kTileM, wchunk, n, g);
  }
}

// Large-M down pass with the row tile resident in LDS: a workgroup of 4 waves takes one 128-row
// tile of the sorted intermediate and kDrChunks consecutive 256-column chunks of the output. The
// tile's whole K (every K-step of the intermediate row, at most kDrMaxSteps) goes global -> LDS
// once, by the same direct loads and swizzle as k_gemm_tile; then each wave runs one K pipeline
// over its chunks' weights (64 columns per chunk), the next step's weight fragments in flight
// while a step multiplies, across chunk boundaries too, and writes a finished chunk's bf16 slot
// rows straight from registers. No barrier after the tile is loaded: the waves share only the
// read-only tile. Against one chunk per workgroup (three K-steps each at intermediate 384) the
// tile is gathered once instead of once per chunk and the pipeline is not drained and refilled
// every three steps. Measured on 8K tokens, hidden 3072, intermediate 384, fp8: down 205 -> 181 us
// (its stores included: without them both passes take ~113 us).
constexpr int kDrChunks = 4;
constexpr int kDrMaxSteps = 4;

inline size_t down_rows_lds_bytes(int nks) { return (size_t)nks * TileLds::bytes; }

template <int WF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_down_rows(GemmParams p, int n_groups, int n_blocks, int sub_shift) {
  using L = TileLds;
  constexpr int MT = kTileM / 16;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  __shared__ __attribute__((aligned(16))) int row_sid[kTileM];
  __shared__ __attribute__((aligned(16))) float row_w[kTileM];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int total = n_groups * n_blocks;
  // unit order as in k_gemm_tile: runs of xcd_run consecutive units per XCD turn, tile-major
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3, run = p.xcd_run;
  const int u = (pos / run) * (8 * run) + xcd * run + pos % run;
  if (u >= total) return;
  const int blk = u / n_groups;
  const int grp = u - blk * n_groups;
  const int r0 = blk * kTileM;
  if (r0 >= *p.num_post_pad) return;
  // 16-row groups holding no slot skip their loads, MFMAs and stores
  const int mtv =
      __builtin_amdgcn_readfirstlane((tile_slots(p.sorted_ids + r0, p.S, lane) + 15) >> 4);
  if (mtv == 0) return;
  const int e = p.block_expert[blk >> sub_shift];
  const int nks = p.NKS;
  const int c0 = grp * kDrChunks;  // first 256-column chunk
  TileRows<1> tr;
  tile_weights<WF, 1>(p, e, (c0 * kTileWaves + wave) * 4, tr);
  if (tid < kTileM) {
    row_sid[tid] = p.sorted_ids[r0 + tid];
    row_w[tid] = p.sorted_w[r0 + tid];
  }
  const v4i ra = rsrc_words(p.a, p.a_bytes);
  const v4i ras = rsrc_words(p.as, p.as_bytes);
  const uint32_t rend = (uint32_t)(r0 + 16 * mtv);
  auto act_row = [&](int r, uint32_t stride) -> uint32_t {
    return (uint32_t)r < rend ? (uint32_t)r * stride : kOutOfRange;
  };
  constexpr bool A4 = a_is_fp4(WF);
  constexpr int kAPitch = A4 ? KSTEP / 2 : kLdsPitch;
  constexpr int kALoads = A4 ? 2 : 4;
  constexpr int kARows = 32 / kALoads;
  uint32_t aoff[kALoads];
#pragma unroll
  for (int j = 0; j < kALoads; ++j) {
    if constexpr (A4) {
      const int lr = lane >> 2;
      aoff[j] = act_row(r0 + 32 * wave + kARows * j + lr, (uint32_t)p.a_stride) +
                16u * ((lane & 3) ^ a4_swz(lr));
    } else {
      aoff[j] = act_row(r0 + 32 * wave + kARows * j + (lane >> 3), (uint32_t)p.a_stride) +
                16u * ((lane & 7) ^ (lane >> 3));
    }
  }
  const uint32_t asoff = wave < 2 ? act_row(r0 + 64 * wave + lane, (uint32_t)p.a_srs) : kOutOfRange;
  const uint32_t lds0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)lds;
  // the whole K of the tile: step ks in stage ks
  for (int ks = 0; ks < nks; ++ks) {
    const uint32_t st = lds0 + ks * L::bytes;
#pragma unroll
    for (int j = 0; j < kALoads; ++j)
      lds_load16(ra, st + L::a + (32 * wave + kARows * j) * kAPitch, aoff[j], ks * kAPitch);
    lds_load4(ras, st + L::as + 256 * wave, asoff, 4 * ks);
  }
  Stage<WF, 1> bs[2];
  load_b<WF, 1, 1>(p, tr, 0, lane, bs[0]);
  wait_loads_barrier<0>();

  const int u0 = A4 ? (g ^ a4_swz(n)) << 4 : (g ^ (n & 7)) << 4;
  const int u1 = ((4 + g) ^ (n & 7)) << 4;
  auto a_frag = [&](int stage, int mt, v8i& a8, uint32_t& sa) {
    const uint8_t* st = lds + stage * L::bytes;
    const uint8_t* base = st + L::a + n * kAPitch;
    a8.lo = *(const v4i*)(base + mt * 16 * kAPitch + u0);
    a8.hi = A4 ? v4i{0, 0, 0, 0} : *(const v4i*)(base + mt * 16 * kAPitch + u1);
    sa = *(const uint32_t*)(st + L::as + 4 * (16 * mt + n));
  };
  v4f acc[MT][4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();
  const int nq = kDrChunks * nks;
  // Step q multiplies K-step ks of chunk c from weight slot q % 2; the weights of step q + 1 go
  // out first. After a chunk's last K-step its rows are stored and the accumulators cleared.
  auto loop = [&](auto MVC) {
    constexpr int MV = decltype(MVC)::value;
    int c = 0, ks = 0;
    auto step = [&](auto SLOT, int q) {
      constexpr int s = decltype(SLOT)::value;
      const bool last_k = ks + 1 == nks;
      if (q + 1 < nq) {
        TileRows<1> tn = tr;
        tn.nt0 = ((c0 + c + (last_k ? 1 : 0)) * kTileWaves + wave) * 4;
        load_b<WF, 1, 1>(p, tn, last_k ? 0 : ks + 1, lane, bs[1 - s]);
      }
      v8i a8[2];
      uint32_t sa[2];
      a_frag(ks, 0, a8[0], sa[0]);
      static_for<MV>([&](auto MTI) {
        constexpr int mt = decltype(MTI)::value;
        if constexpr (mt + 1 < MV) a_frag(ks, mt + 1, a8[(mt + 1) & 1], sa[(mt + 1) & 1]);
        mma_frags<WF>(a8[mt & 1], (int)(sa[mt & 1] >> (8 * g)), bs[s].b, (int)bs[s].sb, acc[mt]);
      });
      if (last_k) {
        epilogue_down_tile(p, acc, (c0 + c) * kTileWaves + wave, n, g, row_sid, row_w, mtv);
        zero_acc();
        ++c;
        ks = 0;
      } else {
        ++ks;
      }
    };
    int q = 0;
    for (; q + 1 < nq; q += 2) {
      step(std::integral_constant<int, 0>{}, q);
      step(std::integral_constant<int, 1>{}, q + 1);
    }
    if (q < nq) step(std::integral_constant<int, 0>{}, q);
  };
  if constexpr (A4 || WF == WF_FP4) {
    if (mtv > 4) loop(std::integral_constant<int, 8>{});
    else if (mtv > 2) loop(std::integral_constant<int, 4>{});
    else if (mtv > 1) loop(std::integral_constant<int, 2>{});
    else loop(std::integral_constant<int, 1>{});
  } else {
    if (mtv > 4) loop(std::integral_constant<int, 8>{});
    else if (mtv > 2) loop(std::integral_constant<int, 4>{});
    else loop(std::integral_constant<int, 2>{});
  }
}

template <int WF, int MT, bool GATE_UP>
__global__ __launch_bounds__(64) void k_gemm_direct(GemmParams p) {
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  const int r0 = blockIdx.y * p.block_m;
  if (r0 >= *p.num_post_pad) return;
  const int e = p.block_expert[blockIdx.y];
  const int r1 = r0 + p.block_m;
  const int chunk = blockIdx.x;
  TileRows<MT> tr;
  tile_weights<WF, MT>(p, e, chunk * 4, tr);
  for (int m0 = r0; m0 < r1; m0 += 16 * MT) {
    tile_act_rows<WF, MT, GATE_UP>(p, m0, r1, n, g, tr);
    v4f acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};
    Stage<WF, MT> cur, nxt;
    load_stage<WF, MT>(p, tr, 0, lane, cur);
    for (int ks = 0; ks < p.NKS; ++ks) {
      if (ks + 1 < p.NKS) load_stage<WF, MT>(p, tr, ks + 1, lane, nxt);
      mma_stage<WF, MT>(cur, 8 * g, acc);
      if (ks + 1 < p.NKS) cur = nxt;
    }
    if (GATE_UP) {
      int hrow[MT][4];
      layout_rows<MT>(m0, r1, g, hrow);
      epilogue_gate_up<WF, MT>(p, acc, hrow, chunk, n);
    }
    else epilogue_down<MT>(p, acc, m0, r1, chunk, n, g);
  }
}

// Most small-M units (column chunks x capacity tiles) for which the stream launcher splits K.
constexpr int kSplitKMaxUnits = 1024;

// Deepest register ring (K-steps in flight per wave) that divides the K-step count: fp8 weights
// 3 stages, fp4 2, bf16 2. For fp4 the shallower ring raises occupancy from three to four waves
// per SIMD; measured on 128 tokens, hidden 3072, intermediate 768: block 125 -> 119 us (4 stages
// against 2; 1 stage 121 us); for fp8 1 to 3 stages give the same time.
inline int stream_depth(int wf, int nks) {
  int dmax = wf == WF_BF16 ? 2 : (wf == WF_FP8 ? 3 : 2);
  const int d = tuning().stream_depth;
  if (d >= 1 && d <= 4) dmax = wf == WF_BF16 ? (d < 2 ? d : 2) : d;
  for (int d = dmax; d > 1; --d)
    if (nks % d == 0) return d;
  return 1;
}

// Pipelined K-steps in the large-M launcher: measured on the 8K-token prefill, gate_up 233 -> 223
// us (fp8) and on 4096 tokens x 512 experts 195 -> 184 us (fp4); down 101 -> 99 us (fp4) but
// 203 -> 205 us (fp8, three K-steps), where it stays off.
// Raised wave priority while a pipelined step issues its MFMAs (the other workgroup on the CU
// does its memory work meanwhile): 8K-token gate_up 204.7 -> 198.3 us; the fp4 down pass went
// 87.2 -> 89.2 us at 4096 tokens x 512 experts, so gate_up only.
inline bool tile_prio(bool gate_up) {
  if (tuning().prio >= 0) return tuning().prio != 0;
  return gate_up;
}

inline bool tile_pipe(bool gate_up, int wf) {
  if (tuning().tile_pipe >= 0) return tuning().tile_pipe != 0;
  return gate_up || w_is_fp4(wf);
}

// n_blocks: the layout's tile capacity, or the expert slots of the slot-order plan
template <int WF, bool GATE_UP, int D, int KS = 1, bool SO = false, int NG = 1>
hipError_t launch_stream(const GemmParams& p, int n_chunks, int n_blocks, hipStream_t st) {
  const int total = n_chunks * n_blocks;
  const int grid = ((total + 7) / 8) * 8;
  if (p.w_nt)
    hipLaunchKernelGGL((k_gemm_stream<WF, 1, GATE_UP, D, KS, kNonTemporal, SO, NG>), dim3(grid),
                       dim3(64 * KS), 0, st, p, n_chunks, n_blocks);
  else
    hipLaunchKernelGGL((k_gemm_stream<WF, 1, GATE_UP, D, KS, 0, SO, NG>), dim3(grid), dim3(64 * KS),
                       0, st, p, n_chunks, n_blocks);
  return hipGetLastError();
}

template <int WF, int D, bool SO = false>
hipError_t launch_down_sa(const GemmParams& p, int n_groups, int n_blocks, hipStream_t st) {
  // the ring's steady loop and its peeled last group assume D divides the K-step count; another
  // depth would run a step past the end of the tile's rows
  if (p.NKS % D != 0) return hipErrorInvalidValue;
  const int total = n_groups * n_blocks;
  const int grid = ((total + 7) / 8) * 8;
  const size_t lds = (size_t)sa_lds_bytes(p.a_stride, p.a_srs);
  if (p.w_nt)
    hipLaunchKernelGGL((k_gemm_down_sa<WF, D, kNonTemporal, SO>), dim3(grid), dim3(64 * kSaWaves),
                       lds, st, p, n_groups, n_blocks);
  else
    hipLaunchKernelGGL((k_gemm_down_sa<WF, D, 0, SO>), dim3(grid), dim3(64 * kSaWaves), lds, st,
                       p, n_groups, n_blocks);
  return hipGetLastError();
}

// The slot-order plan: units over (column chunk, expert slot); the down pass shares its tiles
// across four column chunks where the shape allows, as in the sorted plan.
template <int WF, bool GATE_UP>
hipError_t launch_slot_order(const GemmParams& p, int n_chunks, hipStream_t st) {
  const int ns = p.E + p.so_tiles;
  const int d = stream_depth(WF, p.NKS);
  if constexpr (!GATE_UP && WF != WF_BF16) {
    if (n_chunks % kSaWaves == 0 && sa_lds_bytes(p.a_stride, p.a_srs) <= kSaMaxLds) {
      switch (d) {
        case 4: return launch_down_sa<WF, 4, true>(p, n_chunks / kSaWaves, ns, st);
        case 3: return launch_down_sa<WF, 3, true>(p, n_chunks / kSaWaves, ns, st);
        case 2: return launch_down_sa<WF, 2, true>(p, n_chunks / kSaWaves, ns, st);
        default: return launch_down_sa<WF, 1, true>(p, n_chunks / kSaWaves, ns, st);
      }
    }
  }
  if constexpr (GATE_UP && w_is_fp4(WF)) {
    // fp4 weights: a unit takes two adjacent chunks (one activation stream, 8 KB of weights per
    // K-step as with fp8) with a 3-deep ring where the K-step count allows
    const int pd = tuning().pair_fp4 < 0 ? 3 : tuning().pair_fp4;  // ring depth, 0: off
    if (n_chunks % 2 == 0 && pd == 4 && p.NKS % 4 == 0)
      return launch_stream<WF, GATE_UP, 4, 1, true, 2>(p, n_chunks / 2, ns, st);
    if (n_chunks % 2 == 0 && pd == 3 && p.NKS % 3 == 0)
      return launch_stream<WF, GATE_UP, 3, 1, true, 2>(p, n_chunks / 2, ns, st);
  }
  switch (d) {
    case 4: return launch_stream<WF, GATE_UP, (WF == WF_BF16 ? 1 : 4), 1, true>(p, n_chunks, ns, st);
    case 3: return launch_stream<WF, GATE_UP, (WF == WF_BF16 ? 1 : 3), 1, true>(p, n_chunks, ns, st);
    case 2: return launch_stream<WF, GATE_UP, 2, 1, true>(p, n_chunks, ns, st);
    default: return launch_stream<WF, GATE_UP, 1, 1, true>(p, n_chunks, ns, st);
  }
}

template <int WF, bool GATE_UP>
hipError_t launch_small(const GemmParams& p0, int n_chunks, int n_blocks, hipStream_t st);

template <int WF, bool GATE_UP>
hipError_t launch_one(bool large, const GemmParams& p, int n_blocks, hipStream_t st) {
  const int n_chunks = GATE_UP ? p.I / 32 : p.H / 64;
  if (large) {
    const int n_tile_chunks = n_chunks / kTileWaves;
    const bool tiles = WF != WF_BF16 && n_tile_chunks * kTileWaves == n_chunks &&
                       (p.block_m == kTileM || p.block_m == 2 * kTileM);
    constexpr int W = WF == WF_BF16 ? WF_FP8 : WF;
    // fp8 weights only: with fp4 weights (half the bytes per step) the pass measured slower
    // (4096 tokens x 512 experts, down 80 -> 88 us; W4A4 unchanged)
    if constexpr (WF == WF_FP8 && !GATE_UP) {
    if (tiles && p.combine == 3 && p.NKS <= kDrMaxSteps &&
        n_tile_chunks % kDrChunks == 0 && tuning().down_rows != 0) {
      const int sub_shift = p.block_m == kTileM ? 0 : 1;
      const int n_groups = n_tile_chunks / kDrChunks;
      const int total = n_groups * (n_blocks << sub_shift);
      // default unit order: one contiguous range per XCD (8K tokens: down 181 us with runs of
      // 16 tiles, 172-176 with runs of 4, 8 or 32, 171 with one range)
      GemmParams q = p;
      if (q.xcd_run <= 0) q.xcd_run = (total + 7) / 8;
      const int gq = 8 * q.xcd_run;
      const size_t lds = down_rows_lds_bytes(p.NKS);
      // four K-steps of LDS stages exceed the 64 KiB default: raise the kernel's limit once per
      // device (the attribute belongs to the current device's copy of the kernel)
      if (lds > 65536) {
        static std::atomic<uint64_t> attr_set{0};
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        const uint64_t bit = dev < 64 ? 1ull << dev : 0;
        if (!bit || !(attr_set.load() & bit)) {
          e = hipFuncSetAttribute((const void*)k_down_rows<W>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)down_rows_lds_bytes(kDrMaxSteps));
          if (e != hipSuccess) return e;
          attr_set.fetch_or(bit);
        }
      }
      hipLaunchKernelGGL((k_down_rows<W>), dim3(((total + gq - 1) / gq) * gq), dim3(256), lds, st,
                         q, n_groups, n_blocks << sub_shift, sub_shift);
      return hipGetLastError();
    }
    }
    if (tiles) {
      const int sub_shift = p.block_m == kTileM ? 0 : 1;
      const int total = n_tile_chunks * (n_blocks << sub_shift);
      // default: runs of 4 tiles (all their column chunks); run 0: one contiguous range per XCD
      GemmParams q = p;
      if (q.xcd_run < 0) q.xcd_run = 4 * n_tile_chunks;
      if (q.xcd_run == 0) q.xcd_run = (total + 7) / 8;
      const int gq = 8 * q.xcd_run;  // whole rounds of the unit mapping
      const dim3 grid(((total + gq - 1) / gq) * gq), block(256);
      if (tile_pipe(GATE_UP, WF) && tile_prio(GATE_UP))
        hipLaunchKernelGGL((k_gemm_tile<W, GATE_UP, true, true>), grid, block, 0, st, q,
                           n_tile_chunks, n_blocks << sub_shift, sub_shift);
      else if (tile_pipe(GATE_UP, WF))
        hipLaunchKernelGGL((k_gemm_tile<W, GATE_UP, true>), grid, block, 0, st, q, n_tile_chunks,
                           n_blocks << sub_shift, sub_shift);
      else
        hipLaunchKernelGGL((k_gemm_tile<W, GATE_UP, false>), grid, block, 0, st, q, n_tile_chunks,
                           n_blocks << sub_shift, sub_shift);
    } else {
      hipLaunchKernelGGL((k_gemm_direct<WF, 4, GATE_UP>), dim3(n_chunks, n_blocks), dim3(64), 0, st, p);
    }
    return hipGetLastError();
  }
  if (p.so) return launch_slot_order<WF, GATE_UP>(p, n_chunks, st);
  return launch_small<WF, GATE_UP>(p, n_chunks, n_blocks, st);
}

// Small-M launcher, sorted layout.
template <int WF, bool GATE_UP>
hipError_t launch_small(const GemmParams& p0, int n_chunks, int n_blocks, hipStream_t st) {
  GemmParams p = p0;
  // Few units (a handful of tokens: the capacity holds hardly more tiles than the layout uses):
  // units over the capacity, so none waits for the tile count before its first weight loads.
  if (tuning().cap_units != 0 && p.block_m == 16 && n_chunks * n_blocks <= kSplitKMaxUnits)
    p.cap_units = 1;
  // Split K over 4 waves when the layout has fewer 16-row tiles than a quarter of the SIMDs' share
  // (a handful of tokens) and each wave keeps whole ring groups.
  if (WF != WF_BF16 && p.block_m == 16 && n_chunks * n_blocks <= kSplitKMaxUnits &&
      p.NKS % 4 == 0) {
    switch (stream_depth(WF, p.NKS / 4)) {
      case 4: return launch_stream<WF, GATE_UP, (WF == WF_BF16 ? 1 : 4), 4>(p, n_chunks, n_blocks, st);
      case 3: return launch_stream<WF, GATE_UP, (WF == WF_BF16 ? 1 : 3), 4>(p, n_chunks, n_blocks, st);
      case 2: return launch_stream<WF, GATE_UP, 2, 4>(p, n_chunks, n_blocks, st);
      default: return launch_stream<WF, GATE_UP, 1, 4>(p, n_chunks, n_blocks, st);
    }
  }
  if constexpr (!GATE_UP && WF != WF_BF16) {
    if (p.block_m == 16 && n_chunks % kSaWaves == 0 &&
        sa_lds_bytes(p.a_stride, p.a_srs) <= kSaMaxLds) {
      switch (stream_depth(WF, p.NKS)) {
        case 4: return launch_down_sa<WF, 4>(p, n_chunks / kSaWaves, n_blocks, st);
        case 3: return launch_down_sa<WF, 3>(p, n_chunks / kSaWaves, n_blocks, st);
        case 2: return launch_down_sa<WF, 2>(p, n_chunks / kSaWaves, n_blocks, st);
        default: return launch_down_sa<WF, 1>(p, n_chunks / kSaWaves, n_blocks, st);
      }
    }
  }
  switch (stream_depth(WF, p.NKS)) {
    case 4: return launch_stream<WF, GATE_UP, (WF == WF_BF16 ? 1 : 4)>(p, n_chunks, n_blocks, st);
    case 3: return launch_stream<WF, GATE_UP, (WF == WF_BF16 ? 1 : 3)>(p, n_chunks, n_blocks, st);
    case 2: return launch_stream<WF, GATE_UP, 2>(p, n_chunks, n_blocks, st);
    default: return launch_stream<WF, GATE_UP, 1>(p, n_chunks, n_blocks, st);
  }
}

template <bool GATE_UP>
hipError_t launch_wf(int wf, bool large, const GemmParams& p, int n_blocks, hipStream_t st) {
  if (n_blocks <= 0) return hipSuccess;
  switch (wf) {
    case WF_FP8: return launch_one<WF_FP8, GATE_UP>(large, p, n_blocks, st);
    case WF_FP4: return launch_one<WF_FP4, GATE_UP>(large, p, n_blocks, st);
    case WF_FP4A4: return launch_one<WF_FP4A4, GATE_UP>(large, p, n_blocks, st);
    default: return launch_one<WF_BF16, GATE_UP>(large, p, n_blocks, st);
  }
}

}  // namespace

bool slot_order_fits(int T, int E, int top_k, int I) {
  const int S = T * (top_k + 1), E1 = E + 1;
  return T <= kSlotOrderMaxT && S >= E1 && (size_t)E1 * (I / 32) > (size_t)kSplitKMaxUnits;
}

hipError_t launch_gate_up(int wf, bool large, const GemmParams& p, int n_blocks, hipStream_t st) {
  return launch_wf<true>(wf, large, p, n_blocks, st);
}
hipError_t launch_down(int wf, bool large, const GemmParams& p, int n_blocks, hipStream_t st) {
  return launch_wf<false>(wf, large, p, n_blocks, st);
}

}  // namespace mxmoe
