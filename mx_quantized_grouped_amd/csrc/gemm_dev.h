// Device building blocks of the grouped GEMMs on gfx950 block-scaled MFMA, shared by the
// separate-launch kernels (gemm.hip) and the one-launch decode kernel (fused.hip): operand
// stages, buffer descriptors, weight / activation fragment loads, the MFMA of one K-step, and the
// SwiGLU helpers of the gate_up epilogue.
//
// A wavefront owns 4 weight fragments (64 output columns) of one block_m-row tile of the sorted
// layout, for the whole K. Weight fragments are prepacked so that each wave load is a contiguous
// 1 KiB; activation rows are gathered per lane. MT 16-row tiles share every fragment loaded.
#pragma once
#include <type_traits>
#include <utility>

#include "device.h"
#include "kernels.h"

namespace mxmoe {

template <int WF> struct Frag;
template <> struct Frag<WF_FP8> { static constexpr int bytes = 2048; };
template <> struct Frag<WF_FP4> { static constexpr int bytes = 1024; };
template <> struct Frag<WF_BF16> { static constexpr int bytes = 4096; };
template <> struct Frag<WF_FP4A4> { static constexpr int bytes = 1024; };

// Operands of one 128-K step for one wave: 4 weight fragments and MT activation fragments.
template <int WF, int MT>
struct Stage {
  v4i b[4][WF == WF_BF16 ? 4 : 2];
  v4i a[MT][WF == WF_BF16 ? 4 : 2];
  uint32_t sb;      // byte f: scale of fragment f for this lane's (row, K-block)
  uint32_t sa[MT];  // byte g: scale of K-block 4 ks + g of the lane's row
};

// Buffer descriptor of a raw byte range (gfx9 raw-buffer format word); loads past num_bytes
// return zero, which is how rows outside the tile read as zero without a branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): a loop whose index is a
// compile-time constant in the body (register slots picked by it stay registers).
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

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
  constexpr int FB = Frag<WF>::bytes;
  const size_t wbytes = (size_t)p.NT * p.NKS * FB;
  tr.w = raw_rsrc(p.w + (size_t)e * wbytes, (uint32_t)wbytes);
  if (WF != WF_BF16) {
    const size_t sbytes = (size_t)(p.NT / 4) * p.NKS * 256;
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
    tr.asoff[mt] = ok ? (uint32_t)ar * (uint32_t)p.a_srs : kOutOfRange;
  }
}

// Cache-policy operand of a buffer load: the non-temporal (streaming) hint. The small-M launcher
// reads each weight byte once per call and sets it on its weight loads: measured on the 32-token
// MXFP8 block, gate_up 55.7 -> 49.0 us (5.8 TB/s), down 33.6 -> 30.6 us, block 98.2 -> 87.3 us;
// 128-token MXFP4 block 119.8 -> 112.2 us (the coherence bits sc0 / sc1 alone change nothing). The
// large-M launcher reuses weight slices across an expert's tiles from L2 and keeps the default
// (with the hint, the 8K-token gate_up went 208 -> 270 us).
constexpr int kNonTemporal = 2;

// AUX: cache-policy operand of the weight loads.
template <int WF, int MT, int MTR, int AUX = 0>
__device__ __forceinline__ void load_b(const GemmParams& p, const TileRows<MTR>& tr, int ks,
                                       int lane, Stage<WF, MT>& s) {
  constexpr int FB = Frag<WF>::bytes;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int soff = (((tr.nt0 >> 2) * p.NKS + ks) * 4 + f) * FB;
    const uint32_t vo = 16u * lane;
    if (WF == WF_FP8) {
      s.b[f][0] = __builtin_amdgcn_raw_buffer_load_b128(tr.w, vo, soff, AUX);
      s.b[f][1] = __builtin_amdgcn_raw_buffer_load_b128(tr.w, vo + 1024u, soff, AUX);
    } else if (w_is_fp4(WF)) {
      s.b[f][0] = __builtin_amdgcn_raw_buffer_load_b128(tr.w, vo, soff, AUX);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s.b[f][q] = __builtin_amdgcn_raw_buffer_load_b128(tr.w, vo + 1024u * q, soff, AUX);
    }
  }
  if (WF != WF_BF16)
    s.sb = __builtin_amdgcn_raw_buffer_load_b32(tr.ws, 4u * lane, ((tr.nt0 >> 2) * p.NKS + ks) * 256, AUX);
}

template <int WF, int MT>
__device__ __forceinline__ void load_a(const TileRows<MT>& tr, int ks, Stage<WF, MT>& s) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (a_is_fp4(WF)) {  // one K-block (32 codes, 16 bytes) per lane; rows of 64 bytes per step
      s.a[mt][0] = __builtin_amdgcn_raw_buffer_load_b128(tr.a, tr.aoff[mt], ks * (KSTEP / 2), 0);
      s.sa[mt] = __builtin_amdgcn_raw_buffer_load_b32(tr.as, tr.asoff[mt], 4 * ks, 0);
    } else if (WF != WF_BF16) {
      s.a[mt][0] = __builtin_amdgcn_raw_buffer_load_b128(tr.a, tr.aoff[mt], ks * KSTEP, 0);
      s.a[mt][1] = __builtin_amdgcn_raw_buffer_load_b128(tr.a, tr.aoff[mt] + 64u, ks * KSTEP, 0);
      s.sa[mt] = __builtin_amdgcn_raw_buffer_load_b32(tr.as, tr.asoff[mt], 4 * ks, 0);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s.a[mt][q] = __builtin_amdgcn_raw_buffer_load_b128(tr.a, tr.aoff[mt] + 64u * q,
                                                           ks * KSTEP * 2, 0);
    }
  }
}

template <int WF, int MT, int AUX = 0>
__device__ __forceinline__ void load_stage(const GemmParams& p, const TileRows<MT>& tr, int ks,
                                           int lane, Stage<WF, MT>& s) {
  load_b<WF, MT, MT, AUX>(p, tr, ks, lane, s);
  load_a<WF, MT>(tr, ks, s);
}

// The four block-scaled MFMAs of one A fragment against the wave's 4 weight fragments; the scale
// operand of fragment F is byte F of sb (selected by the instruction's op_sel). The element
// formats go in the instruction's cbsz (A) and blgp (B) fields: 0 E4M3, 4 E2M1; an E2M1 operand
// is 32 codes in the low four dwords of the lane.
template <int WF, int F = 0>
__device__ __forceinline__ void mma_frags(const v8i& a8, int sa, const v4i (&b)[4][2], int sb,
                                          v4f (&acc)[4]) {
  if constexpr (F < 4) {
    v8i b8;
    b8.lo = b[F][0];
    b8.hi = (WF == WF_FP8) ? b[F][1] : v4i{0, 0, 0, 0};
    acc[F] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        a8, b8, acc[F], a_is_fp4(WF) ? 4 : 0, w_is_fp4(WF) ? 4 : 0, 0, sa, F, sb);
    mma_frags<WF, F + 1>(a8, sa, b, sb, acc);
  }
}

// ash = 8 * (lane / 16): the lane's K-block byte within the A scale dword.
template <int WF, int MT>
__device__ __forceinline__ void mma_stage(const Stage<WF, MT>& s, int ash, v4f (&acc)[MT][4]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if constexpr (WF != WF_BF16) {
      v8i a8;
      a8.lo = s.a[mt][0];
      a8.hi = a_is_fp4(WF) ? v4i{0, 0, 0, 0} : s.a[mt][1];
      mma_frags<WF>(a8, (int)(s.sa[mt] >> ash), s.b, (int)s.sb, acc[mt]);
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[mt][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf, s.a[mt][q]), __builtin_bit_cast(v8bf, s.b[f][q]),
              acc[mt][f], 0, 0, 0);
    }
  }
}

// SiLU with the hardware reciprocal (about 1 ulp); exp overflow for very negative g gives
// g * rcp(inf) = -0, the limit.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Maximum of non-negative finite values over the 16 lanes of a DPP row (lanes 16r .. 16r + 15), in
// every lane of the row: the row of an MFMA result fragment, i.e. one 16-column slice of four
// output rows. Non-negative floats order like their bit patterns, so the reduction runs on
// unsigned integers, one DPP-sourced max per step (a float maximum also canonicalises each
// operand: two extra instructions per step). Every source lane lies inside the row, so the
// bound control never applies.
__device__ __forceinline__ float row16_max(float v) {
  uint32_t u = __float_as_uint(v);
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:4, row_ror:8
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x124, 0xF, 0xF, true));
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, true));
  return __uint_as_float(u);
}

}  // namespace mxmoe
