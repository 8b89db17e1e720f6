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

template <int WF, int MT>
__device__ __forceinline__ void load_b(const GemmParams& p, const TileRows<MT>& tr, int ks,
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
  load_b<WF, MT>(p, tr, ks, lane, s);
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
      float* orow = p.combine == 1 ? p.out32 + (size_t)sid * p.H
                                   : p.out32 + (size_t)(sid / p.k1) * p.H;
      const int c0 = 64 * chunk + n;
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
    for (int s = 0; s < D; ++s) load_b<WF, MT>(p, tr, s, lane, buf[s]);
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
    hipLaunchKernelGGL((k_gemm_direct<WF, 4, GATE_UP>), dim3(n_chunks, n_blocks), dim3(64), 0, st, p);
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
