// Router gate in front of the routing step: logits[t, e] = sum_h x[t, h] * w_gate[e, h], bf16
// operands on bf16 MFMA with fp32 accumulation — the bf16 gate of "Ling-3.0-flash: Tối ưu hóa độ
// trễ giải mã lên 54% trên 4 GPU Blackwell" ("Sửa thước đo trước khi sửa máy"), whose 2.6 MB
// gate-weight kernel took 7 us with its weights in L2 and 11 us with them cold there.
//
// A workgroup of 4 waves computes a (16 TM)-token x (16 F)-expert tile. The waves split the K-steps
// of 32 (wave w takes steps w, w + 4, ...), and their partial sums are added in LDS in wave order,
// so the result does not depend on timing. Each wave keeps 4 (or, for tiles of more than 4
// fragments, 2) K-steps of loads in flight. Each load instruction reads 64 bytes of each of 16
// rows (the MFMA operand layout). The tile grows with the batch (measured, hidden 3072 and 128
// experts unless stated): one fragment up to 256 tokens (the weight stream spread over the most
// CUs: 7.1 us for 32 tokens, 7.4 us for 128, against 9.7 us with 16 x 32 tiles); 16 x 32 up to
// 1024 tokens (10.1 us at 1024). Beyond, and beyond 256 tokens from 512 experts on, the tiles are
// staged through LDS (k_gate_lds: whole cache lines per load instead of 64-byte row segments):
// 32 x 64 up to 4096 tokens (2048 tokens: 12.0 us against 18.3 us for 16 x 32), 64 x 32 beyond
// (8192 tokens: 19.6 us; 26.5 us for the best register tile, 64 x 64; 56 us for 16 x 64, which
// re-reads the weights for every 16 tokens). With 512 experts, hidden 2048: 32 x 64 up to 1024
// tokens (9.4 us against 23.7 us for 16 x 32), 64 x 64 beyond (4096 tokens: 19.8 us; 28.8 us for
// the best register tile, 64 x 128). Loading more K-steps ahead in the register tiles changed
// nothing. Every tile gives the same logits: wave w always takes K-steps w, w + 4, ... and the
// partial sums are added in wave order.
#include <cstdlib>

#include "device.h"
#include "kernels.h"

namespace mxmoe {

namespace {

constexpr int kGateRows = 16;
constexpr int kGateWaves = 4;
constexpr int kGateDepth = 4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t gate_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// OUT_F32: fp32 logits, else bf16 (round to nearest even). Rows past T and experts past E read as
// zero (buffer range checks) and are not stored.
// TM 16-token fragments x F 16-expert fragments per workgroup.
template <int TM, int F, bool OUT_F32>
__global__ __launch_bounds__(256) void k_gate(const uint16_t* x, const uint16_t* wg, int T, int H,
                                              int E, void* out) {
  __shared__ v4f part[kGateWaves][TM * F][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * (kGateRows * TM), e0 = blockIdx.y * (16 * F);
  const uint32_t row_bytes = (uint32_t)H * 2u;
  const int tr = min(kGateRows * TM, T - t0), er = min(16 * F, E - e0);
  const auto ra = gate_rsrc(x + (size_t)t0 * H, (uint32_t)tr * row_bytes);
  const auto rb = gate_rsrc(wg + (size_t)e0 * H, (uint32_t)er * row_bytes);
  // lane (n, g) holds K elements 8 g .. 8 g + 7 of a step: row n of the token fragment, row n of
  // each expert fragment
  const uint32_t aoff = (uint32_t)n * row_bytes + 16u * g;
  const int nsteps = H / 32;
  v4f acc[TM][F];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int f = 0; f < F; ++f) acc[m][f] = v4f{0.f, 0.f, 0.f, 0.f};
  constexpr int D = TM * F > 4 ? 2 : kGateDepth;  // K-steps of loads in flight per wave
  for (int k0 = wave; k0 < nsteps; k0 += kGateWaves * D) {
    v4i a[D][TM], b[D][F];
#pragma unroll
    for (int d = 0; d < D; ++d) {  // every load of the batch before the first MFMA
      // steps past the end load out of range: zeros, so the MFMAs below need no branch (a branch
      // let the compiler sink each load next to its use)
      const int k = k0 + kGateWaves * d;
      const uint32_t oob = k < nsteps ? 0u : 0x80000000u;
      const int soff = (k < nsteps ? k : 0) * 64;
#pragma unroll
      for (int m = 0; m < TM; ++m)
        a[d][m] = __builtin_amdgcn_raw_buffer_load_b128(ra, (aoff + 16u * m * row_bytes) | oob,
                                                        soff, 0);
#pragma unroll
      for (int f = 0; f < F; ++f)
        b[d][f] = __builtin_amdgcn_raw_buffer_load_b128(rb, (aoff + 16u * f * row_bytes) | oob,
                                                        soff, 0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int f = 0; f < F; ++f)
          acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[d][m]),
                                                              __builtin_bit_cast(v8bf, b[d][f]),
                                                              acc[m][f], 0, 0, 0);
    }
  }
  // C[4 g + i][n] of token fragment m, expert fragment f; fragment j = m * F + f is stored by wave
  // j % 4 after adding the waves' partial sums in wave order
  auto store = [&](int j, const v4f& v) {
    const int m = j / F, f = j - m * F;
    const int e = e0 + 16 * f + n;
    if (e >= E) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * m + 4 * g + i;
      if (t >= T) continue;
      if (OUT_F32) ((float*)out)[(size_t)t * E + e] = v[i];
      else ((uint16_t*)out)[(size_t)t * E + e] = (uint16_t)f32_to_bf16_bits(v[i]);
    }
  };
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int f = 0; f < F; ++f) part[wave][m * F + f][lane] = acc[m][f];
  __syncthreads();
  for (int j = wave; j < TM * F; j += kGateWaves) {
    v4f s = part[0][j][lane];
#pragma unroll
    for (int w = 1; w < kGateWaves; ++w) {
      const v4f q = part[w][j][lane];
      s[0] += q[0]; s[1] += q[1]; s[2] += q[2]; s[3] += q[3];
    }
    store(j, s);
  }
}

// LDS-staged variant: chunks of 128 K elements (256 bytes of each row) of the x and W_g tiles are
// loaded row-contiguously (16 consecutive lanes cover one row's 256 bytes, so every load touches
// whole cache lines), written to LDS (row pitch 272 bytes: the 16 rows of a fragment read fall in
// different banks), and each wave reads its MFMA fragments of K-step w of the chunk from there.
// Two LDS stages; the next chunk's global loads are in flight while the current one is multiplied.
constexpr int kGateChunkBytes = 256;
constexpr int kGatePitch = kGateChunkBytes + 16;

template <int TM, int F, bool OUT_F32>
__global__ __launch_bounds__(256) void k_gate_lds(const uint16_t* x, const uint16_t* wg, int T,
                                                  int H, int E, void* out) {
  constexpr int XR = 16 * TM, WR = 16 * F;                  // tile rows of x and of W_g
  constexpr int XP = XR * kGateChunkBytes / 16 / 256;        // 16-byte pieces per thread
  constexpr int WP = WR * kGateChunkBytes / 16 / 256;
  constexpr int STAGE = (XR + WR) * kGatePitch;
  constexpr int PART = kGateWaves * TM * F * 64 * 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE > PART ? 2 * STAGE : PART];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * XR, e0 = blockIdx.y * WR;
  const uint32_t row_bytes = (uint32_t)H * 2u;
  const int tr = min(XR, T - t0), er = min(WR, E - e0);
  const auto ra = gate_rsrc(x + (size_t)t0 * H, (uint32_t)tr * row_bytes);
  const auto rb = gate_rsrc(wg + (size_t)e0 * H, (uint32_t)er * row_bytes);
  const int nchunks = (int)((row_bytes + kGateChunkBytes - 1) / kGateChunkBytes);
  v4i rx[XP], rw[WP];
  // piece q = tid + 256 i: row q / 16, bytes 16 (q % 16) of the chunk; bytes past the row end
  // read as zero (out-of-range offset)
  auto load = [&](int c) {
    const uint32_t kb = (uint32_t)c * kGateChunkBytes + 16u * (tid & 15);
    const uint32_t oob = kb < row_bytes ? 0u : 0x80000000u;
#pragma unroll
    for (int i = 0; i < XP; ++i)
      rx[i] = __builtin_amdgcn_raw_buffer_load_b128(
          ra, ((uint32_t)((tid >> 4) + 16 * i) * row_bytes + kb) | oob, 0, 0);
#pragma unroll
    for (int i = 0; i < WP; ++i)
      rw[i] = __builtin_amdgcn_raw_buffer_load_b128(
          rb, ((uint32_t)((tid >> 4) + 16 * i) * row_bytes + kb) | oob, 0, 0);
  };
  auto store = [&](int st) {
    uint8_t* base = lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < XP; ++i)
      *(v4i*)(base + ((tid >> 4) + 16 * i) * kGatePitch + 16 * (tid & 15)) = rx[i];
#pragma unroll
    for (int i = 0; i < WP; ++i)
      *(v4i*)(base + (XR + (tid >> 4) + 16 * i) * kGatePitch + 16 * (tid & 15)) = rw[i];
  };
  v4f acc[TM][F];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int f = 0; f < F; ++f) acc[m][f] = v4f{0.f, 0.f, 0.f, 0.f};
  load(0);
  store(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) load(c + 1);
    const uint8_t* base = lds + (c & 1) * STAGE;
    // wave w: K-step w of the chunk, lane (n, g) K elements 8 g .. 8 g + 7 of row n
    const int co = 64 * wave + 16 * g;
    v4i a[TM], b[F];
#pragma unroll
    for (int m = 0; m < TM; ++m) a[m] = *(const v4i*)(base + (16 * m + n) * kGatePitch + co);
#pragma unroll
    for (int f = 0; f < F; ++f) b[f] = *(const v4i*)(base + (XR + 16 * f + n) * kGatePitch + co);
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int f = 0; f < F; ++f)
        acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[m]),
                                                            __builtin_bit_cast(v8bf, b[f]),
                                                            acc[m][f], 0, 0, 0);
    if (more) store((c + 1) & 1);
    __syncthreads();
  }
  // partial sums of the 4 waves (one K-step of each chunk each) added in wave order
  v4f* part = (v4f*)lds;
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int f = 0; f < F; ++f) part[(wave * TM * F + m * F + f) * 64 + lane] = acc[m][f];
  __syncthreads();
  for (int j = wave; j < TM * F; j += kGateWaves) {
    v4f sum = part[j * 64 + lane];
#pragma unroll
    for (int w = 1; w < kGateWaves; ++w) {
      const v4f q = part[(w * TM * F + j) * 64 + lane];
      sum[0] += q[0]; sum[1] += q[1]; sum[2] += q[2]; sum[3] += q[3];
    }
    const int m = j / F, f = j - m * F;
    const int e = e0 + 16 * f + n;
    if (e >= E) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * m + 4 * g + i;
      if (t >= T) continue;
      if (OUT_F32) ((float*)out)[(size_t)t * E + e] = sum[i];
      else ((uint16_t*)out)[(size_t)t * E + e] = (uint16_t)f32_to_bf16_bits(sum[i]);
    }
  }
}

template <int TM, int F>
hipError_t launch_gate_lds(const uint16_t* x, const uint16_t* wg, int T, int H, int E, bool f32,
                           void* out, hipStream_t st) {
  const dim3 grid((T + 16 * TM - 1) / (16 * TM), (E + 16 * F - 1) / (16 * F));
  const dim3 block(256);
  if (f32) hipLaunchKernelGGL((k_gate_lds<TM, F, true>), grid, block, 0, st, x, wg, T, H, E, out);
  else hipLaunchKernelGGL((k_gate_lds<TM, F, false>), grid, block, 0, st, x, wg, T, H, E, out);
  return hipGetLastError();
}

template <int TM, int F>
hipError_t launch_gate_f(const uint16_t* x, const uint16_t* wg, int T, int H, int E, bool f32,
                         void* out, hipStream_t st) {
  const dim3 grid((T + kGateRows * TM - 1) / (kGateRows * TM), (E + 16 * F - 1) / (16 * F));
  const dim3 block(256);
  if (f32) hipLaunchKernelGGL((k_gate<TM, F, true>), grid, block, 0, st, x, wg, T, H, E, out);
  else hipLaunchKernelGGL((k_gate<TM, F, false>), grid, block, 0, st, x, wg, T, H, E, out);
  return hipGetLastError();
}

}  // namespace

bool valid_gate_tile(int tile) {
  switch (tile) {
    case 11: case 12: case 14: case 21: case 22: case 24: case 28: case 41: case 42: case 44:
    case 48: case 84: case 124: case 142: case 144: case 148: return true;
    default: return false;
  }
}

hipError_t launch_gate(const uint16_t* x, const uint16_t* wg, int T, int H, int E, bool f32,
                       void* out, int tile, hipStream_t st) {
  // tile: 10 * TM + F for register tiles, 100 + 10 * TM + F for LDS-staged ones; 0 = by shape
  int cfg = T <= 256 ? 11
            : E >= 512 ? (T <= 1024 ? 124 : 144)
                       : (T <= 1024 ? 12 : (T <= 4096 ? 124 : 142));
  if (tile) cfg = tile;
  else if (valid_gate_tile(tuning().gate_tile)) cfg = tuning().gate_tile;
  switch (cfg) {
    case 11: return launch_gate_f<1, 1>(x, wg, T, H, E, f32, out, st);
    case 12: return launch_gate_f<1, 2>(x, wg, T, H, E, f32, out, st);
    case 14: return launch_gate_f<1, 4>(x, wg, T, H, E, f32, out, st);
    case 22: return launch_gate_f<2, 2>(x, wg, T, H, E, f32, out, st);
    case 24: return launch_gate_f<2, 4>(x, wg, T, H, E, f32, out, st);
    case 28: return launch_gate_f<2, 8>(x, wg, T, H, E, f32, out, st);
    case 42: return launch_gate_f<4, 2>(x, wg, T, H, E, f32, out, st);
    case 44: return launch_gate_f<4, 4>(x, wg, T, H, E, f32, out, st);
    case 48: return launch_gate_f<4, 8>(x, wg, T, H, E, f32, out, st);
    case 84: return launch_gate_f<8, 4>(x, wg, T, H, E, f32, out, st);
    case 144: return launch_gate_lds<4, 4>(x, wg, T, H, E, f32, out, st);
    case 148: return launch_gate_lds<4, 8>(x, wg, T, H, E, f32, out, st);
    case 124: return launch_gate_lds<2, 4>(x, wg, T, H, E, f32, out, st);
    case 142: return launch_gate_lds<4, 2>(x, wg, T, H, E, f32, out, st);
    case 21: return launch_gate_f<2, 1>(x, wg, T, H, E, f32, out, st);
    case 41: return launch_gate_f<4, 1>(x, wg, T, H, E, f32, out, st);
    default: return launch_gate_f<1, 4>(x, wg, T, H, E, f32, out, st);
  }
}

}  // namespace mxmoe
