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
// A wavefront owns 4 weight fragments (64 output columns) of one block_m-row tile of the sorted
// layout, for the whole K. Weight fragments are prepacked so that each wave load is a contiguous
// 1 KiB; activation rows are gathered per lane. MT 16-row tiles share every fragment loaded.
//
// Small-M launcher (decode): one wave per (column chunk, tile); D K-steps of operands are in flight
// per wave (a register ring), since at decode M the weights are read once and HBM latency is the
// limit. Units are ordered so that the tiles of one expert on one column chunk are consecutive on
// the same XCD (workgroups go round-robin over the 8 XCDs, each with its own L2): an expert with
// more than one tile reads its weights from HBM once, the grouped-MoE program ordering of the
// MiniMax-M3 page's local-shapes passage.
#include <cstdlib>

#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

template <int WF> struct Frag;
template <> struct Frag<WF_FP8> { static constexpr int bytes = 2048; };
template <> struct Frag<WF_FP4> { static constexpr int bytes = 1024; };
template <> struct Frag<WF_BF16> { static constexpr int bytes = 4096; };

// Operands of one 128-K step for one wave: 4 weight fragments and MT activation fragments.
template <int WF, int MT>
struct Stage {
  v4i b[4][WF == WF_BF16 ? 4 : 2];
  v4i a[MT][WF == WF_BF16 ? 4 : 2];
  uint32_t sb[4];
  uint32_t sa[MT];
};

// Buffer descriptor of a raw byte range (gfx9 raw-buffer format word); loads past num_bytes
// return zero, which is how rows outside the tile read as zero without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;

// Per-wave view of its tile: descriptors of the expert's weights / scales and of the activation
// rows, the lane's byte offset into its A row (per 16-row tile mt) and the wave's first fragment.
template <int MT>
struct TileRows {
  __amdgpu_buffer_rsrc_t w, ws, a, as;
  uint32_t aoff[MT];
  uint32_t asoff[MT];
  int nt0;
};

// Weight and activation descriptors of the wave's tile (expert e, first fragment nt0).
template <int WF, int MT>
__device__ __forceinline__ void tile_weights(const GemmParams& p, int e, int nt0, TileRows<MT>& tr) {
  constexpr int FB = WF == WF_FP8 ? 2048 : (WF == WF_FP4 ? 1024 : 4096);
  const size_t wbytes = (size_t)p.NT * p.NKS * FB;
  tr.w = raw_rsrc(p.w + (size_t)e * wbytes, (uint32_t)wbytes);
  if (WF != WF_BF16) {
    const size_t sbytes = (size_t)p.NT * p.NKG * 256;
    tr.ws = raw_rsrc(p.ws + (size_t)e * sbytes, (uint32_t)sbytes);
    tr.as = raw_rsrc(p.as, p.as_bytes);
  }
  tr.a = raw_rsrc(p.a, p.a_bytes);
  tr.nt0 = nt0;
}

// The lane's activation row per 16-row tile: gate_up gathers the token row of each slot (rows
// whose slot is padding read as zero); down reads the sorted intermediate rows in place (padding
// rows hold zeros written by gate_up), so it needs no lookup.
template <int WF, int MT, bool GATE_UP>
__device__ __forceinline__ void tile_act_rows(const GemmParams& p, int m0, int r1, int n, int g,
                                              TileRows<MT>& tr) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = m0 + 16 * mt + n;
    bool ok;
    int ar;
    if (GATE_UP) {
      const int sid = r < r1 ? p.sorted_ids[r] : p.S;
      ok = sid < p.S;
      ar = sid / p.k1;
    } else {
      ok = r < r1;
      ar = r;
    }
    tr.aoff[mt] = ok ? (uint32_t)ar * (uint32_t)p.a_stride + 16u * g : kOutOfRange;
    tr.asoff[mt] = ok ? (uint32_t)ar * (uint32_t)p.a_srs + 4u * g : kOutOfRange;
  }
}

template <int WF, int MT, int MTR>
__device__ __forceinline__ void load_b(const GemmParams& p, const TileRows<MTR>& tr, int ks,
                                       int lane, Stage<WF, MT>& s) {
  constexpr int FB = Frag<WF>::bytes;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int soff = ((tr.nt0 + f) * p.NKS + ks) * FB;
    const uint32_t vo = 16u * lane;
    if (WF == WF_FP8) {
      s.b[f][0] = __builtin_amdgcn_raw_buffer_load_b128(tr.w, vo, soff, 0);
      s.b[f][1] = __builtin_amdgcn_raw_buffer_load_b128(tr.w, vo + 1024u, soff, 0);
    } else if (WF == WF_FP4) {
      s.b[f][0] = __builtin_amdgcn_raw_buffer_load_b128(tr.w, vo, soff, 0);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s.b[f][q] = __builtin_amdgcn_raw_buffer_load_b128(tr.w, vo + 1024u * q, soff, 0);
    }
    if (WF != WF_BF16)
      s.sb[f] = __builtin_amdgcn_raw_buffer_load_b32(tr.ws, 4u * lane,
                                                     ((tr.nt0 + f) * p.NKG + (ks >> 2)) * 256, 0);
  }
}

template <int WF, int MT>
__device__ __forceinline__ void load_a(const TileRows<MT>& tr, int ks, Stage<WF, MT>& s) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (WF != WF_BF16) {
      s.a[mt][0] = __builtin_amdgcn_raw_buffer_load_b128(tr.a, tr.aoff[mt], ks * KSTEP, 0);
      s.a[mt][1] = __builtin_amdgcn_raw_buffer_load_b128(tr.a, tr.aoff[mt] + 64u, ks * KSTEP, 0);
      s.sa[mt] = __builtin_amdgcn_raw_buffer_load_b32(tr.as, tr.asoff[mt], 16 * (ks >> 2), 0);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s.a[mt][q] = __builtin_amdgcn_raw_buffer_load_b128(tr.a, tr.aoff[mt] + 64u * q,
                                                           ks * KSTEP * 2, 0);
    }
  }
}

template <int WF, int MT>
__device__ __forceinline__ void load_stage(const GemmParams& p, const TileRows<MT>& tr, int ks,
                                           int lane, Stage<WF, MT>& s) {
  load_b<WF, MT, MT>(p, tr, ks, lane, s);
  load_a<WF, MT>(tr, ks, s);
}

template <int WF, int MT>
__device__ __forceinline__ void mma_stage(const Stage<WF, MT>& s, int ks, v4f (&acc)[MT][4]) {
  const int sh = 8 * (ks & 3);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (WF != WF_BF16) {
        v8i a8, b8;
        a8.lo = s.a[mt][0];
        a8.hi = s.a[mt][1];
        b8.lo = s.b[f][0];
        b8.hi = (WF == WF_FP8) ? s.b[f][1] : v4i{0, 0, 0, 0};
        acc[mt][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a8, b8, acc[mt][f], 0, WF == WF_FP4 ? 4 : 0, 0, (int)(s.sa[mt] >> sh), 0,
            (int)(s.sb[f] >> sh));
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[mt][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf, s.a[mt][q]), __builtin_bit_cast(v8bf, s.b[f][q]),
              acc[mt][f], 0, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// acc[mt][f][i] is C[row 4g+i of tile mt][column n of fragment f]. Fragments 0/1 are gate/up of
// intermediate columns chunk*32 + 0..15, fragments 2/3 of chunk*32 + 16..31.
template <int WF, int MT>
__device__ __forceinline__ void epilogue_gate_up(const GemmParams& p, const v4f (&acc)[MT][4],
                                                 int m0, int r1, int chunk, int n, int g) {
  const int ic0 = 32 * chunk;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = m0 + 16 * mt + 4 * g + i;
      float a0 = silu(acc[mt][0][i]) * acc[mt][1][i];
      float a1 = silu(acc[mt][2][i]) * acc[mt][3][i];
      if (WF != WF_BF16) {
        float m = fmaxf(fabsf(a0), fabsf(a1));
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        int se = mx_shared_exp<8>(m);
        if (rr < r1) {
          uint8_t* hr = p.h + (size_t)rr * p.h_stride + ic0;
          hr[n] = (uint8_t)e4m3_code(a0, se);
          hr[16 + n] = (uint8_t)e4m3_code(a1, se);
          if (n == 0) p.hs[(size_t)rr * p.h_srs + act_scale_byte(chunk)] = (uint8_t)(se + 127);
        }
      } else if (rr < r1) {
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
        const int rr = m0 + 16 * mt + 4 * g + i;
        if (rr >= r1) continue;
        if (WF != WF_BF16) {
          for (int c = p.I + n; c < p.Ip; c += 16) p.h[(size_t)rr * p.h_stride + c] = 0;
          if (n == 0)
            for (int kb = p.I / 32; kb < p.Ip / 32; ++kb)
              p.hs[(size_t)rr * p.h_srs + act_scale_byte(kb)] = 127;
        } else {
          uint16_t* hr = (uint16_t*)(p.h + (size_t)rr * p.h_stride);
          for (int c = p.I + n; c < p.Ip; c += 16) hr[c] = 0;
        }
      }
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
      const float wt = p.topk_w[sid];
      const int c0 = 64 * chunk + n;
      if (p.combine == 3) {
        uint16_t* orow = (uint16_t*)p.out32 + (size_t)sid * p.H;
#pragma unroll
        for (int f = 0; f < 4; ++f) orow[c0 + 16 * f] = (uint16_t)f32_to_bf16_bits(wt * acc[mt][f][i]);
        continue;
      }
      float* orow = p.combine == 1 ? p.out32 + (size_t)sid * p.H
                                   : p.out32 + (size_t)(sid / p.k1) * p.H;
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        float v = wt * acc[mt][f][i];
        if (p.combine == 1) orow[c0 + 16 * f] = v;
        else atomicAdd(orow + c0 + 16 * f, v);
      }
    }
  }
}

// ------------------------------------------------------------------------------ small-M
template <int WF, int MT, bool GATE_UP, int D>
__global__ __launch_bounds__(64) void k_gemm_stream(GemmParams p, int n_chunks, int n_blocks) {
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  // Unit order: XCD x = blockIdx % 8 takes the x-th contiguous range of units; units run
  // chunk-major, tiles fastest, so the tiles of one expert on one chunk share an XCD.
  const int total = n_chunks * n_blocks;
  const int per_xcd = (total + 7) >> 3;
  const int u = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (u >= total) return;
  const int chunk = u / n_blocks, blk = u - chunk * n_blocks;
  const int r0 = blk * p.block_m;
  if (r0 >= *p.num_post_pad) return;
  const int e = p.block_expert[blk];
  const int r1 = r0 + p.block_m;
  TileRows<MT> tr;
  tile_weights<WF, MT>(p, e, chunk * 4, tr);
  for (int m0 = r0; m0 < r1; m0 += 16 * MT) {
    v4f acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};
    // Register ring of D stages; the host picks D dividing NKS, so the steady-state loop issues
    // the loads of group k0 + D while multiplying group k0 without any branch, and the last group
    // is peeled. Weight loads of the first group go out before the (dependent) row lookup.
    Stage<WF, MT> buf[D];
#pragma unroll
    for (int s = 0; s < D; ++s) load_b<WF, MT, MT>(p, tr, s, lane, buf[s]);
    tile_act_rows<WF, MT, GATE_UP>(p, m0, r1, n, g, tr);
#pragma unroll
    for (int s = 0; s < D; ++s) load_a<WF, MT>(tr, s, buf[s]);
    int k0 = 0;
    for (; k0 + D < p.NKS; k0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        mma_stage<WF, MT>(buf[s], k0 + s, acc);
        load_stage<WF, MT>(p, tr, k0 + s + D, lane, buf[s]);
      }
    }
#pragma unroll
    for (int s = 0; s < D; ++s) mma_stage<WF, MT>(buf[s], k0 + s, acc);
    if (GATE_UP) epilogue_gate_up<WF, MT>(p, acc, m0, r1, chunk, n, g);
    else epilogue_down<MT>(p, acc, m0, r1, chunk, n, g);
  }
}

// ------------------------------------------------------------------------------ large-M
// Prefill launcher: a workgroup of 4 waves computes a 128-row x 256-column tile (rows of one expert
// from the sorted layout). The gathered activation tile of each 128-K step is staged through LDS
// (double-buffered) and shared by the 4 waves; each wave streams its own 4 weight fragments (64
// columns) into registers, one K-step ahead. Per K-step a wave issues 8 x 4 block-scaled MFMAs.
// LDS rows are 128 bytes with the eight 16-byte column units of row r stored at unit c ^ (r & 7):
// the 16 rows an MFMA operand read touches then spread over all banks (measured on gfx950: ~198
// B/clk/CU for this read pattern, against ~119 with 16-byte row padding).
constexpr int kTileM = 128;
constexpr int kTileWaves = 4;
constexpr int kLdsPitch = KSTEP;
__device__ __forceinline__ int lds_unit(int row, int c) { return (c ^ (row & 7)) << 4; }

template <int WF, bool GATE_UP, int P>
__global__ __launch_bounds__(256) void k_gemm_tile(GemmParams p, int n_chunks, int n_blocks) {
  constexpr int MT = kTileM / 16;
  // per buffer: the 128 x 128-byte activation tile, then the tile's scale bytes for the K-step's
  // group (16 bytes per row: the four lane-group dwords of the kernel-native scale layout)
  constexpr int kTileBytes = kTileM * kLdsPitch;
  constexpr int kBufBytes = kTileBytes + kTileM * 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kBufBytes];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  // wave-uniform by construction; readfirstlane tells the compiler, so scalar buffer offsets that
  // depend on it stay in SGPRs (otherwise every buffer load becomes a per-lane waterfall loop)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Unit order: each XCD takes a contiguous range of units, tile-major with the column chunks of a
  // tile adjacent — the gathered activation tile is fetched once into that XCD's L2 and reused by
  // its column chunks, and an expert's consecutive tiles reuse its weight slices from L2.
  const int total = n_chunks * n_blocks;
  const int per_xcd = (total + 7) >> 3;
  const int u = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (u >= total) return;
  const int blk = u / n_chunks, chunk = u - blk * n_chunks;
  const int r0 = blk * kTileM;
  if (r0 >= *p.num_post_pad) return;
  const int e = p.block_expert[blk];
  const int r1 = r0 + kTileM;
  const int wchunk = chunk * kTileWaves + wave;  // this wave's 64-column chunk

  TileRows<MT> tr;
  tile_weights<WF, MT>(p, e, wchunk * 4, tr);
  // Copy assignment: 8 consecutive lanes move one row's 128-byte K-step segment (a full cache
  // line per 8 lanes); thread t handles rows 32q + t/8 (q = 0..3), 16-byte unit t % 8.
  // Threads t < 128 also move row t's 16 scale bytes of the K-step's group.
  const int cunit = tid & 7, crow0 = tid >> 3;
  uint32_t coff[4], csoff = kOutOfRange;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = r0 + 32 * q + crow0;
    bool ok = true;
    int ar = r;
    if (GATE_UP) {
      const int sid = p.sorted_ids[r];
      ok = sid < p.S;
      ar = sid / p.k1;
    }
    coff[q] = ok ? (uint32_t)ar * (uint32_t)p.a_stride + 16u * cunit : kOutOfRange;
  }
  if (tid < kTileM) {
    const int r = r0 + tid;
    bool ok = true;
    int ar = r;
    if (GATE_UP) {
      const int sid = p.sorted_ids[r];
      ok = sid < p.S;
      ar = sid / p.k1;
    }
    csoff = ok ? (uint32_t)ar * (uint32_t)p.a_srs : kOutOfRange;
  }

  v4f acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};

  // P-deep register ring: the weight fragments, the activation bytes and scale bytes this thread
  // copies into LDS for K-step ks + P are requested while step ks is multiplied; LDS is
  // double-buffered (step ks + 1 is written while step ks is read).
  Stage<WF, 1> bst[P];
  v4i ca[P][4];
  v4i cs[P];
  auto load_copy = [&](int ks, int slot) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      ca[slot][q] = __builtin_amdgcn_raw_buffer_load_b128(tr.a, coff[q], ks * KSTEP, 0);
    if (tid < kTileM) cs[slot] = __builtin_amdgcn_raw_buffer_load_b128(tr.as, csoff, 16 * (ks >> 2), 0);
  };
  auto store_copy = [&](int slot, int buf) {
    uint8_t* dst = lds[buf];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 32 * q + crow0;
      *(v4i*)(dst + row * kLdsPitch + lds_unit(row, cunit)) = ca[slot][q];
    }
    if (tid < kTileM) *(v4i*)(dst + kTileBytes + 16 * tid) = cs[slot];
  };
  auto load_all = [&](int ks, int slot) {
    load_b<WF, 1, MT>(p, tr, ks, lane, bst[slot]);
    load_copy(ks, slot);
  };
  auto compute = [&](int ks, int buf, const Stage<WF, 1>& b) {
    const int sh = 8 * (ks & 3);
    // rows n + 16 mt share (row & 7) = n & 7, so the swizzled units are loop-invariant
    const uint8_t* base = lds[buf] + n * kLdsPitch;
    const uint8_t* sbase = lds[buf] + kTileBytes + 16 * n + 4 * g;
    const int u0 = lds_unit(n, g), u1 = lds_unit(n, 4 + g);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v8i a8;
      a8.lo = *(const v4i*)(base + mt * 16 * kLdsPitch + u0);
      a8.hi = *(const v4i*)(base + mt * 16 * kLdsPitch + u1);
      const uint32_t sa = *(const uint32_t*)(sbase + 256 * mt);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        v8i b8;
        b8.lo = b.b[f][0];
        b8.hi = (WF == WF_FP8) ? b.b[f][1] : v4i{0, 0, 0, 0};
        acc[mt][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a8, b8, acc[mt][f], 0, WF == WF_FP4 ? 4 : 0, 0, (int)(sa >> sh), 0,
            (int)(b.sb[f] >> sh));
      }
    }
  };

  if constexpr (P == 1) {
    // single-step ring: next step's loads go out before this step's multiply; separate weight
    // registers for the current and the next step
    Stage<WF, 1> bnx;
    load_all(0, 0);
    store_copy(0, 0);
    __syncthreads();
    for (int ks = 0; ks < p.NKS; ++ks) {
      const bool more = ks + 1 < p.NKS;
      if (more) {
        load_b<WF, 1, MT>(p, tr, ks + 1, lane, bnx);
        load_copy(ks + 1, 0);
      }
      compute(ks, ks & 1, bst[0]);
      if (more) store_copy(0, (ks + 1) & 1);
      __syncthreads();
      if (more) bst[0] = bnx;
    }
  } else {
    // P divides NKS (host-checked), so every load in the steady-state loop is in range
#pragma unroll
    for (int s = 0; s < P; ++s) load_all(s, s);
    store_copy(0, 0);
    __syncthreads();
    int k0 = 0;
    for (; k0 + P < p.NKS; k0 += P) {
#pragma unroll
      for (int s = 0; s < P; ++s) {
        const int ks = k0 + s;
        compute(ks, ks & 1, bst[s]);
        store_copy((s + 1) % P, (ks + 1) & 1);  // step ks + 1 (ks + 1 < NKS here)
        load_all(ks + P, s);
        __syncthreads();
      }
    }
#pragma unroll
    for (int s = 0; s < P; ++s) {  // last group: no further loads
      const int ks = k0 + s;
      compute(ks, ks & 1, bst[s]);
      if (s + 1 < P) store_copy(s + 1, (ks + 1) & 1);
      __syncthreads();
    }
  }

  if (GATE_UP) epilogue_gate_up<WF, MT>(p, acc, r0, r1, wchunk, n, g);
  else epilogue_down<MT>(p, acc, r0, r1, wchunk, n, g);
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
      mma_stage<WF, MT>(cur, ks, acc);
      if (ks + 1 < p.NKS) cur = nxt;
    }
    if (GATE_UP) epilogue_gate_up<WF, MT>(p, acc, m0, r1, chunk, n, g);
    else epilogue_down<MT>(p, acc, m0, r1, chunk, n, g);
  }
}

// Deepest register ring (K-steps in flight per wave) that divides the K-step count and keeps two
// waves per SIMD: fp8 weights fit 3 stages, fp4 4, bf16 2.
inline int stream_depth(int wf, int nks) {
  int dmax = wf == WF_BF16 ? 2 : (wf == WF_FP8 ? 3 : 4);
  if (const char* env = getenv("MXMOE_STREAM_DEPTH")) {  // A/B knob: 1..4
    int d = atoi(env);
    if (d >= 1 && d <= 4) dmax = wf == WF_BF16 ? (d < 2 ? d : 2) : d;
  }
  for (int d = dmax; d > 1; --d)
    if (nks % d == 0) return d;
  return 1;
}

template <int WF, bool GATE_UP, int D>
hipError_t launch_stream(const GemmParams& p, int n_chunks, int n_blocks, hipStream_t st) {
  const int total = n_chunks * n_blocks;
  const int grid = ((total + 7) / 8) * 8;
  hipLaunchKernelGGL((k_gemm_stream<WF, 1, GATE_UP, D>), dim3(grid), dim3(64), 0, st, p, n_chunks,
                     n_blocks);
  return hipGetLastError();
}

template <int WF, bool GATE_UP>
hipError_t launch_one(bool large, const GemmParams& p, int n_blocks, hipStream_t st) {
  const int n_chunks = GATE_UP ? p.I / 32 : p.H / 64;
  if (large) {
    const int n_tile_chunks = n_chunks / kTileWaves;
    if (WF != WF_BF16 && p.block_m == kTileM && n_tile_chunks * kTileWaves == n_chunks) {
      const int total = n_tile_chunks * n_blocks;
      const dim3 grid(((total + 7) / 8) * 8), block(256);
      constexpr int W = WF == WF_BF16 ? WF_FP8 : WF;
      // ring depth: 2 K-steps when it divides the step count (3 would spill), else 1
      if (p.NKS % 2 == 0)
        hipLaunchKernelGGL((k_gemm_tile<W, GATE_UP, 2>), grid, block, 0, st, p, n_tile_chunks, n_blocks);
      else
        hipLaunchKernelGGL((k_gemm_tile<W, GATE_UP, 1>), grid, block, 0, st, p, n_tile_chunks, n_blocks);
    } else {
      hipLaunchKernelGGL((k_gemm_direct<WF, 4, GATE_UP>), dim3(n_chunks, n_blocks), dim3(64), 0, st, p);
    }
    return hipGetLastError();
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
    default: return launch_one<WF_BF16, GATE_UP>(large, p, n_blocks, st);
  }
}

}  // namespace

hipError_t launch_gate_up(int wf, bool large, const GemmParams& p, int n_blocks, hipStream_t st) {
  return launch_wf<true>(wf, large, p, n_blocks, st);
}
hipError_t launch_down(int wf, bool large, const GemmParams& p, int n_blocks, hipStream_t st) {
  return launch_wf<false>(wf, large, p, n_blocks, st);
}

}  // namespace mxmoe
