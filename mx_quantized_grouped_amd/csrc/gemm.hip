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
// Work decomposition: one wavefront per (N chunk of 4 fragments = 64 columns, work unit). The
// small-M (decode) launcher makes the work unit a touched expert and loops over all its rows, so
// every weight byte leaves HBM once; the large-M (prefill) launcher makes it a block_m-row tile of
// the sorted layout (the split by M of the same page's local-shapes passage). Each wave streams
// its weight fragments straight from HBM into registers (prepacked so every wave load is a
// contiguous 1 KiB) and gathers its activation rows itself; MT 16-row tiles share every weight
// fragment it loads. The next K-step's operands are loaded before the current one is multiplied.
#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

template <int WF> struct Frag;
template <> struct Frag<WF_FP8> { static constexpr int bytes = 2048; };
template <> struct Frag<WF_FP4> { static constexpr int bytes = 1024; };
template <> struct Frag<WF_BF16> { static constexpr int bytes = 4096; };

// Operands of one K-step (128 K) for one wave.
template <int WF, int MT>
struct Stage {
  // MX: b[f] 8 dwords (fp4 uses the low 4), a[mt] 8 dwords. bf16: 4 x 4 dwords each.
  v4i b[4][WF == WF_BF16 ? 4 : 2];
  v4i a[MT][WF == WF_BF16 ? 4 : 2];
  uint32_t sb[4];
  uint32_t sa[MT];
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

template <int WF, int MT, bool GATE_UP, bool LARGE>
__global__ __launch_bounds__(64) void k_gemm(GemmParams p) {
  constexpr int FB = Frag<WF>::bytes;
  constexpr bool MX = WF != WF_BF16;
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;

  int e, r0, r1;
  if (LARGE) {
    r0 = blockIdx.y * p.block_m;
    if (r0 >= *p.num_post_pad) return;
    e = p.block_expert[blockIdx.y];
    r1 = r0 + p.block_m;
  } else {
    if ((int)blockIdx.y >= *p.n_touched) return;
    e = p.touched[blockIdx.y];
    r0 = p.expert_off[e];
    r1 = p.expert_off[e + 1];
  }
  const int nt0 = blockIdx.x * 4;
  const uint8_t* wb = p.w + ((size_t)e * p.NT + nt0) * (size_t)p.NKS * FB;
  const uint8_t* wsb = MX ? p.ws + ((size_t)e * p.NT + nt0) * (size_t)p.NKG * 256 + lane * 4 : nullptr;

  for (int m0 = r0; m0 < r1; m0 += 16 * MT) {
    const uint8_t* arow[MT];
    const uint8_t* asrow[MT];
    bool aval[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      int r = m0 + 16 * mt + n;
      int sid = r < r1 ? p.sorted_ids[r] : p.S;
      aval[mt] = sid < p.S;
      int ar = aval[mt] ? (GATE_UP ? sid / p.k1 : r) : 0;
      arow[mt] = p.a + (size_t)ar * p.a_stride;
      asrow[mt] = MX ? p.as + (size_t)ar * p.a_srs + 4 * g : nullptr;
    }

    auto load = [&](int ks, Stage<WF, MT>& s) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint8_t* fp = wb + ((size_t)f * p.NKS + ks) * FB + 16 * lane;
        if (WF == WF_FP8) {
          s.b[f][0] = *(const v4i*)fp;
          s.b[f][1] = *(const v4i*)(fp + 1024);
        } else if (WF == WF_FP4) {
          s.b[f][0] = *(const v4i*)fp;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) s.b[f][q] = *(const v4i*)(fp + 1024 * q);
        }
        if (MX) s.sb[f] = *(const uint32_t*)(wsb + ((size_t)f * p.NKG + (ks >> 2)) * 256);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (MX) {
          const uint8_t* ap = arow[mt] + ks * KSTEP + 16 * g;
          s.a[mt][0] = aval[mt] ? *(const v4i*)ap : v4i{0, 0, 0, 0};
          s.a[mt][1] = aval[mt] ? *(const v4i*)(ap + 64) : v4i{0, 0, 0, 0};
          s.sa[mt] = aval[mt] ? *(const uint32_t*)(asrow[mt] + 16 * (ks >> 2)) : 0x7F7F7F7Fu;
        } else {
          const uint8_t* ap = arow[mt] + (size_t)ks * KSTEP * 2 + 16 * g;
#pragma unroll
          for (int q = 0; q < 4; ++q) s.a[mt][q] = aval[mt] ? *(const v4i*)(ap + 64 * q) : v4i{0, 0, 0, 0};
        }
      }
    };

    v4f acc[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};

    Stage<WF, MT> cur, nxt;
    load(0, cur);
    for (int ks = 0; ks < p.NKS; ++ks) {
      if (ks + 1 < p.NKS) load(ks + 1, nxt);
      const int sh = 8 * (ks & 3);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (MX) {
            v8i a8, b8;
            a8.lo = cur.a[mt][0]; a8.hi = cur.a[mt][1];
            b8.lo = cur.b[f][0];
            b8.hi = (WF == WF_FP8) ? cur.b[f][1] : v4i{0, 0, 0, 0};
            acc[mt][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a8, b8, acc[mt][f], 0, WF == WF_FP4 ? 4 : 0, 0, (int)(cur.sa[mt] >> sh), 0,
                (int)(cur.sb[f] >> sh));
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[mt][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(v8bf, cur.a[mt][q]), __builtin_bit_cast(v8bf, cur.b[f][q]),
                  acc[mt][f], 0, 0, 0);
          }
        }
      }
      if (ks + 1 < p.NKS) cur = nxt;
    }

    // ------------------------------------------------------------------ epilogues
    // acc[mt][f][i] is C[row 4g+i of tile mt][column n of fragment f].
    if (GATE_UP) {
      const int ic0 = 32 * blockIdx.x;  // first intermediate column of this wave
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = m0 + 16 * mt + 4 * g + i;
          float a0 = silu(acc[mt][0][i]) * acc[mt][1][i];  // fragments 0/1: gate/up, cols 0..15
          float a1 = silu(acc[mt][2][i]) * acc[mt][3][i];  // fragments 2/3: gate/up, cols 16..31
          if (MX) {
            float m = fmaxf(fabsf(a0), fabsf(a1));
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
            int se = mx_shared_exp<8>(m);
            if (rr < r1) {
              uint8_t* hr = p.h + (size_t)rr * p.h_stride + ic0;
              hr[n] = (uint8_t)e4m3_code(a0, se);
              hr[16 + n] = (uint8_t)e4m3_code(a1, se);
              if (n == 0) p.hs[(size_t)rr * p.h_srs + act_scale_byte(blockIdx.x)] = (uint8_t)(se + 127);
            }
          } else if (rr < r1) {
            uint16_t* hr = (uint16_t*)(p.h + (size_t)rr * p.h_stride) + ic0;
            hr[n] = (uint16_t)f32_to_bf16_bits(a0);
            hr[16 + n] = (uint16_t)f32_to_bf16_bits(a1);
          }
        }
      }
      // K padding of the intermediate (I not a multiple of 128): zero codes, finite scales.
      if (p.Ip > p.I && blockIdx.x == gridDim.x - 1) {
        for (int mt = 0; mt < MT; ++mt)
          for (int i = 0; i < 4; ++i) {
            const int rr = m0 + 16 * mt + 4 * g + i;
            if (rr >= r1) continue;
            if (MX) {
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
    } else {
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
          const int c0 = 64 * blockIdx.x + n;
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            float v = wt * acc[mt][f][i];
            if (p.combine == 1) orow[c0 + 16 * f] = v;
            else atomicAdd(orow + c0 + 16 * f, v);
          }
        }
      }
    }
  }
}

template <int WF, bool GATE_UP>
hipError_t launch_one(bool large, const GemmParams& p, int grid_y, hipStream_t st) {
  dim3 grid(GATE_UP ? p.I / 32 : p.H / 64, grid_y), block(64);
  if (large)
    hipLaunchKernelGGL((k_gemm<WF, 4, GATE_UP, true>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((k_gemm<WF, 2, GATE_UP, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

template <bool GATE_UP>
hipError_t launch_wf(int wf, bool large, const GemmParams& p, int grid_y, hipStream_t st) {
  if (grid_y <= 0) return hipSuccess;
  switch (wf) {
    case WF_FP8: return launch_one<WF_FP8, GATE_UP>(large, p, grid_y, st);
    case WF_FP4: return launch_one<WF_FP4, GATE_UP>(large, p, grid_y, st);
    default: return launch_one<WF_BF16, GATE_UP>(large, p, grid_y, st);
  }
}

}  // namespace

hipError_t launch_gate_up(int wf, bool large, const GemmParams& p, int grid_y, hipStream_t st) {
  return launch_wf<true>(wf, large, p, grid_y, st);
}
hipError_t launch_down(int wf, bool large, const GemmParams& p, int grid_y, hipStream_t st) {
  return launch_wf<false>(wf, large, p, grid_y, st);
}

}  // namespace mxmoe
