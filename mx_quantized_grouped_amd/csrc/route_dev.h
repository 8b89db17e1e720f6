// Device side of the token -> expert top-k router: one wavefront routes one token.
//
// Selection compares an order-preserving key per expert: the logit's bit pattern mapped to an
// unsigned integer that increases with the value (-0 folded onto +0), then the complemented expert
// index. The wave-wide maximum of that key is the largest logit, ties going to the lowest index —
// the fixed tie-break of the routing table. For bf16 logits the whole key fits 32 bits (16-bit
// value key, 16-bit index); fp32 logits compare the 32-bit value key first and the index second.
// The wave maximum uses DPP row operations and two row broadcasts (a handful of VALU cycles) rather
// than LDS permutes. The shared expert then takes slot top_k with weight 1: the folding of the
// shared expert into the routing table described in "Lần theo điểm nghẽn: Tối ưu MiniMax M3 trên
// AMD Instinct MI355X" (shared-expert passage, Fig. 4). Weights are softmax over the selected
// logits (renormalised top-k), computed in fp32.
#pragma once
#include "device.h"

namespace mxmoe {

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadPerm1032 = 0xB1;  // quad_perm:[1,0,3,2]
constexpr int kDppQuadPerm2301 = 0x4E;  // quad_perm:[2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Unsigned maximum over the 64 lanes of the wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  auto step = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppQuadPerm1032, 0xF, 0xF, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppQuadPerm2301, 0xF, 0xF, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowRor4, 0xF, 0xF, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowRor8, 0xF, 0xF, false));
  // every lane now holds its row's maximum; carry rows 0 -> 1 and 2 -> 3, then rows 0..1 -> 2..3
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowBcast15, 0xA, 0xF, false));
  v = step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over the 64 lanes of the wave, returned to every lane (same DPP pattern; rows outside a
// broadcast's row mask add zero).
__device__ __forceinline__ float wave_sum_f32(float v) {
  auto add = [](float x, int y) { return x + __int_as_float(y); };
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppQuadPerm1032, 0xF, 0xF, false));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppQuadPerm2301, 0xF, 0xF, false));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor4, 0xF, 0xF, false));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowRor8, 0xF, 0xF, false));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast15, 0xA, 0xF, false));
  v = add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), kDppRowBcast31, 0xC, 0xF, false));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ uint32_t route_order_key(uint32_t u) {
  if ((u & 0x7FFFFFFFu) == 0) u = 0;  // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float route_key_value(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// Order keys of token t's logits held by this lane (E <= 64 * NPER); experts past E get key 0,
// below every real key.
template <bool F32, int NPER>
__device__ __forceinline__ void route_load_keys(const void* logits, int t, int E, int lane,
                                                uint32_t (&vkey)[NPER]) {
#pragma unroll
  for (int c = 0; c < NPER; ++c) {
    vkey[c] = 0;
    int e = lane + 64 * c;
    if (e < E) {
      if (F32) {
        vkey[c] = route_order_key(((const uint32_t*)logits)[(size_t)t * E + e]);
      } else {
        uint32_t u = (uint32_t)((const uint16_t*)logits)[(size_t)t * E + e] << 16;
        vkey[c] = (route_order_key(u) & 0xFFFF0000u) | (0xFFFFu - (uint32_t)e);  // value | ~index
      }
    }
  }
}

// Top-k selection, weights and the shared slot for token t from its keys; writes the ids/w rows of
// width top_k + 1 and, where ids_lds / w_lds are not null, the same rows to LDS too. Called by all
// 64 lanes.
template <bool F32, int NPER>
__device__ void route_select(uint32_t (&vkey)[NPER], int t, int E, int top_k, int lane,
                             int32_t* ids, float* w, int32_t* ids_lds, float* w_lds) {
  uint32_t mine_v = 0, mine_e = 0;  // lane j keeps the j-th selection
  for (int j = 0; j < top_k; ++j) {
    uint32_t lbest = 0;
#pragma unroll
    for (int c = 0; c < NPER; ++c) lbest = vkey[c] > lbest ? vkey[c] : lbest;
    const uint32_t bv = wave_max_u32(lbest);
    uint32_t be;
    if (F32) {
      // among the experts holding the best value, the lowest index: expert lane + 64 c, so the
      // lowest column with a match and its lowest lane, from one ballot per column (scalar bit
      // scans instead of a second wave reduction)
      be = 0;
#pragma unroll
      for (int c = NPER - 1; c >= 0; --c) {
        const uint64_t m = __ballot(vkey[c] == bv);
        if (m) be = 64u * (uint32_t)c + (uint32_t)__builtin_ctzll(m);
      }
    } else {
      be = 0xFFFFu - (bv & 0xFFFFu);
    }
#pragma unroll
    for (int c = 0; c < NPER; ++c)
      if ((uint32_t)(lane + 64 * c) == be) vkey[c] = 0;  // exactly one lane holds expert be
    if (lane == j) {
      mine_v = bv;
      mine_e = be;
    }
  }
  float v = F32 ? route_key_value(mine_v)
                : __uint_as_float(__float_as_uint(route_key_value(mine_v & 0xFFFF0000u)) & 0xFFFF0000u);
  const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float p = lane < top_k ? expf(v - v0) : 0.f;
  const float s = wave_sum_f32(p);
  const int k1 = top_k + 1;
  int32_t id = -1;
  float wt = 0.f;
  if (lane < top_k) {
    id = (int32_t)mine_e;
    wt = p / s;
  } else if (lane == top_k) {
    id = E;  // shared expert
    wt = 1.0f;
  }
  if (lane < k1) {
    ids[(size_t)t * k1 + lane] = id;
    w[(size_t)t * k1 + lane] = wt;
    if (ids_lds) ids_lds[t * k1 + lane] = id;
    if (w_lds) w_lds[t * k1 + lane] = wt;
  }
}

// Routes tokens t0, t0 + stride, ... (< T) on one wave. The logits of up to 8 tokens are loaded
// before any is selected, so their load latencies overlap instead of adding up.
template <bool F32, int NPER>
__device__ void route_tokens(const void* logits, int t0, int stride, int T, int E, int top_k,
                             int lane, int32_t* ids, float* w, int32_t* ids_lds, float* w_lds) {
  constexpr int B = NPER <= 2 ? 8 : (NPER <= 4 ? 4 : (NPER <= 8 ? 2 : 1));  // <= 16 key registers
  for (int tb = t0; tb < T; tb += B * stride) {
    uint32_t keys[B][NPER];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int t = tb + b * stride;
      if (t < T) route_load_keys<F32, NPER>(logits, t, E, lane, keys[b]);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int t = tb + b * stride;
      if (t < T) route_select<F32, NPER>(keys[b], t, E, top_k, lane, ids, w, ids_lds, w_lds);
    }
  }
}

// route_tokens with the smallest keys-per-lane count that covers E.
template <bool F32>
__device__ __forceinline__ void route_tokens_any(const void* logits, int t0, int stride, int T,
                                                 int E, int top_k, int lane, int32_t* ids,
                                                 float* w, int32_t* ids_lds,
                                                 float* w_lds = nullptr) {
  if (E <= 64) route_tokens<F32, 1>(logits, t0, stride, T, E, top_k, lane, ids, w, ids_lds, w_lds);
  else if (E <= 128) route_tokens<F32, 2>(logits, t0, stride, T, E, top_k, lane, ids, w, ids_lds, w_lds);
  else if (E <= 256) route_tokens<F32, 4>(logits, t0, stride, T, E, top_k, lane, ids, w, ids_lds, w_lds);
  else if (E <= 512) route_tokens<F32, 8>(logits, t0, stride, T, E, top_k, lane, ids, w, ids_lds, w_lds);
  else route_tokens<F32, 16>(logits, t0, stride, T, E, top_k, lane, ids, w, ids_lds, w_lds);
}

}  // namespace mxmoe
