// Internal launch interface between the C ABI (api.hip) and the kernels. Host code only.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxmoe {

constexpr int kMaxTopK = 63;      // one wave holds the selected experts, lane top_k the shared slot
constexpr int kMaxExperts = 1024; // routed experts; E + 1 <= 2048 for the block-wide scans
constexpr int kAlignSmallMaxSlots = 4096;
constexpr int kAlignChunk = 1024; // slots per workgroup in the multi-workgroup sort
// Buffers addressed through 32-bit offsets (buffer descriptors, row offsets) stay below 2 GiB; the
// out-of-range sentinel 0x80000000 must never be a valid offset.
constexpr size_t kMaxBufferBytes = (size_t)1 << 31;

// A/B switches of the measurements behind the kernels' defaults, read from the environment once
// (at the library's first call); -1 = unset, the library's own choice. They never change a result
// beyond the documented variants (unit orders, cache hints, pipelining, tile shapes).
struct Tuning {
  bool trace;          // MXMOE_TRACE: print the plan of every forward call
  int w_nt;            // MXMOE_W_NT: non-temporal weight loads of the small-M launcher (0/1)
  int xcd_order;       // MXMOE_XCD_ORDER: small-M unit order, 1 per-XCD ranges, 0 linear
  int xcd_run_gu;      // MXMOE_XCD_RUN_GU / _DN: large-M run of units per XCD turn
  int xcd_run_dn;      //   (0 one range per XCD, 1 linear); -1 unset
  int stream_depth;    // MXMOE_STREAM_DEPTH: small-M register ring depth 1..4
  int prio;            // MXMOE_PRIO: raised wave priority during the large-M MFMAs (0/1)
  int tile_pipe;       // MXMOE_TILE_PIPE: pipelined large-M K-steps (0/1)
  int slot_order;      // MXMOE_SLOT_ORDER: 0 = automatic plans never take the slot-order plan
  int cap_units;       // MXMOE_CAP_UNITS: 0 = few-unit sorted plans decode units from the tile count
  int final_nt;        // MXMOE_NT: non-temporal slot-row loads of the final sum (0/1)
  int gate_tile;       // MXMOE_GATE_TILE: router gate tile (10 TM + F, +100 LDS-staged)
  int down_rows;       // MXMOE_DOWN_ROWS: 0 = large-M down pass one chunk per workgroup
  int pair_fp4;        // MXMOE_PAIR_FP4: ring depth (3, 4) of paired fp4 gate_up units, 0 off
  int pf_steps;        // MXMOE_PF_STEPS: K-steps of gate_up weights prefetched (0 off)
  int pf_wgs;          // MXMOE_PF_WGS: prefetch workgroups per XCD
};
const Tuning& tuning();

// route.hip
// gate.hip
// tile: 0 = chosen by shape; otherwise one of the tiles valid_gate_tile accepts
bool valid_gate_tile(int tile);
hipError_t launch_gate(const uint16_t* x, const uint16_t* w_gate, int T, int H, int E, bool out_f32,
                       void* logits, int tile, hipStream_t st);

hipError_t launch_route(const void* logits, bool logits_f32, int T, int E, int top_k,
                        int32_t* ids, float* w, hipStream_t st);

// align.hip
struct AlignOut {
  int32_t* sorted_ids;
  int32_t* block_expert;
  int32_t* num_post_pad;
  int32_t* expert_off;  // may be null
  int32_t* touched;     // may be null
  int32_t* n_touched;   // may be null
  // optional: the routing weight of each sorted row (topk_w[sorted_ids[r]], 0 for padding), so the
  // down pass reads a row's weight by row index instead of through its slot id
  const float* topk_w;  // null: no sorted_w
  float* sorted_w;
};
size_t align_scratch_bytes(int T, int E, int top_k);
hipError_t launch_align(const int32_t* ids, int T, int E, int top_k, int block_m,
                        const AlignOut& o, void* scratch, hipStream_t st);

// prologue.hip: route + sort + activation quantisation (or accumulator clearing) for forward.
struct PrologueArgs {
  const void* logits;
  int T, E, top_k;
  int32_t* ids;
  float* w;
  int block_m, cap;
  AlignOut out;
  const uint16_t* x;
  int H;
  uint8_t* xq;      // null: no quantisation (bf16 path)
  uint8_t* xs;
  bool a4;          // E2M1 activation codes (rows of H / 2 bytes), else E4M3 (rows of H bytes)
  int srs;
  float* zero_out;  // null: nothing to clear
  int32_t* zero_cnt;  // n_cnt counters to clear (null: none)
  int n_cnt;
  bool no_sort;     // slot-order plan: routing and quantisation only
  // Prefetch of the slot-order gate_up weights (pf_w null: none): workgroups on each XCD load the
  // first pf_steps K-steps of the units that XCD's gate_up workgroups will run (units over
  // pf_chunks column chunks x pf_nb expert slots, contiguous per-XCD ranges), while the routing
  // runs. gate_up's fetched bytes are unchanged by it (so not L2 hits); its gain comes from the
  // memory-side cache or warm address translations.
  const uint8_t* pf_w;
  const uint8_t* pf_ws;
  size_t pf_wbytes, pf_sbytes;  // per expert: prepacked weight and scale bytes
  int pf_chunks, pf_nb, pf_nks, pf_step_bytes, pf_steps, pf_wgs;
};
hipError_t launch_prologue(const PrologueArgs& a, bool logits_f32, void* align_scratch,
                           hipStream_t st);

// quant.hip
// Canonical MX quantisation (codes row-major, scales [rows, K/32]).
hipError_t launch_quantize_canonical(const void* src, bool src_f32, int rows, int K, bool fp4,
                                     uint8_t* codes, uint8_t* scales, hipStream_t st);

// prepack.hip
struct PrepackDims {
  int E1;      // experts incl. shared
  int N;       // rows per expert (2I for w13, H for w2)
  int K;       // reduction length (H for w13, I for w2)
  int wf;      // WF_FP8 / WF_FP4 / WF_BF16
  bool w13;    // interleave gate/up 16-row tiles
  int I;       // for the w13 interleave
};
size_t prepack_code_bytes(const PrepackDims& d);
size_t prepack_scale_bytes(const PrepackDims& d);
hipError_t launch_prepack(const PrepackDims& d, const void* codes, const uint8_t* scales,
                          void* codes_p, void* scales_p, hipStream_t st);

// gemm.hip
struct GemmParams {
  const uint8_t* a;          // A rows: MX codes or bf16
  const uint8_t* as;         // A kernel-native scales (MX)
  int a_stride;              // bytes per A row
  int a_srs;                 // bytes per A scale row
  uint32_t a_bytes;          // size of the A matrix (rows * a_stride), < 2 GiB
  uint32_t as_bytes;         // size of the A scale matrix
  const uint8_t* w;          // prepacked weights
  const uint8_t* ws;         // prepacked weight scales (MX)
  int NT, NKS;               // per expert: 16-row N tiles, K-steps of 128
  const int32_t* sorted_ids;
  const int32_t* expert_off;
  const int32_t* touched;
  const int32_t* n_touched;
  const int32_t* block_expert;
  const int32_t* num_post_pad;
  int block_m, S, k1;
  // gate_up epilogue
  uint8_t* h;                // intermediate rows [cap, Ip] (MXFP8 codes or bf16)
  uint8_t* hs;               // intermediate scales [cap, h_srs]
  int h_stride, h_srs, I, Ip;
  // down epilogue
  const float* topk_w;
  const float* sorted_w;     // routing weight of each sorted row (0 for padding rows)
  float* out32;              // slot rows [S, H] or token rows [T, H]
  int H;
  int combine;               // 1 fp32 slot rows, 2 fp32 atomics, 3 bf16 slot rows
  // fused final rounding (small-M launcher with the atomic combine): y != null; chunk_done holds
  // one completion counter per 64-column chunk, cleared by the prologue
  uint16_t* y;
  int32_t* chunk_done;
  int T;
  // small-M launcher: 1 units in contiguous per-XCD ranges, 0 plain linear order over the grid
  int xcd_order;
  // large-M launcher: each XCD takes runs of xcd_run consecutive units in turn (1: plain linear
  // order over the grid; 0: one contiguous range per XCD; -1: the launcher's default)
  int xcd_run;
  int w_nt;  // small-M launcher: weight loads with the non-temporal hint
  // small-M launcher, sorted layout with few units: units over the layout's capacity in plain
  // order (a unit whose tile holds no expert, block_expert -1, ends at once), so no unit waits
  // for the tile count before its first weight loads
  int cap_units;
  // Slot-order plan (small-M launcher, no sort): so != 0. A unit is (column chunk, expert slot):
  // slots [0, E) are the routed experts, slots [E, E + so_tiles) the shared expert's tiles of 16
  // consecutive tokens. Every expert owns so_cap = T intermediate rows (expert-major, row
  // e * so_cap + i for its i-th slot in slot order). gate_up's units find a routed expert's slots
  // by a scan of topk_ids, and its chunk-0 unit records them in so_list[e * so_cap + i] (p.S past
  // the count) and their count in so_cnt[e], which the down pass reads instead of scanning again.
  int so, so_tiles, so_cap, E;
  int so_spec;  // down: weight loads before the expert's count is known (few experts without rows)
  const int32_t* topk_ids;
  int32_t* so_list;
  int32_t* so_cnt;
};
// Most tokens of a slot-order plan (rows of one expert, held in LDS by each unit).
constexpr int kSlotOrderMaxT = 256;
// Prefetch of the slot-order gate_up weights in the prologue (fp8 weights): K-steps per unit
// and workgroups per XCD. Measured at 32 tokens, hidden 3072, 128 experts (block, two repeats):
// off 82.7-83.1 us; 2 steps over 32 workgroups 81.6-82.3 (prologue +1.3, gate_up -3 us); 2, 4, 16,
// 64 and 128 workgroups 126, 103, 85, 83-84 and 83-84 us (the prefetch workgroups' dispatch and
// per-CU load rate extend the prologue); 1 step 82-83, 3 steps 83-85. With MXFP4 weights (128
// tokens) no gain, so fp8 only.
constexpr int kPrefetchSteps = 2;
constexpr int kPrefetchWgs = 32;
// Most intermediate bytes (T rows per expert) the automatic choice gives a slot-order plan.
constexpr size_t kSlotOrderMaxRowBytes = 64u << 20;
// Whether the small-M plan of this shape runs in slot order: enough slots that most experts have
// rows (a unit of an empty expert only scans the ids), at most kSlotOrderMaxT tokens, and enough
// gate_up units that K is not split.
bool slot_order_fits(int T, int E, int top_k, int I);
hipError_t launch_gate_up(int wf, bool large, const GemmParams& p, int grid_y, hipStream_t st);
hipError_t launch_down(int wf, bool large, const GemmParams& p, int grid_y, hipStream_t st);

// fused.hip: the whole block for small batches in one launch (routing, layout, gate_up, down and
// the final sum as roles of one grid). Its control words sit at the start of every workspace.
constexpr size_t kFusedCtlBytes = 72 * 1024;  // zero before the first call; every call resets them
constexpr int kFusedBitmapWords = 2560;       // per-expert slot bitmaps of the layout workgroup
constexpr int kFusedMaxFin = 16384;           // final-sum counters: (H / 64) * ceil(T / 8)
constexpr int kFusedMaxT = 128;
constexpr int kFusedDefaultSpin = 50000;      // polls (each ~1 us) before a wait gives up
constexpr size_t kFusedStatusByte = 16;       // offset of the status word in the control words
struct FusedArgs {
  const uint16_t* x;      // bf16 [T, H]
  const void* logits;     // [T, E]
  bool logits_f32;
  const uint8_t* w13;     // prepacked weights and scales
  const uint8_t* s13;
  const uint8_t* w2;
  const uint8_t* s2;
  uint16_t* y;            // bf16 [T, H]
  int T, H, E, top_k, I, Ip;
  int32_t* ids;           // [T, k + 1] routing table
  float* tw;
  AlignOut lay;           // the 16-row sorted layout (every field set)
  int cap;
  uint8_t* xq;            // activation codes [T, H] and scales [T, srs_H], for inspection
  uint8_t* xs;
  int srs_H;
  uint8_t* h;             // intermediate rows [cap, h_stride] and scales [cap, srs_I]
  uint8_t* hs;
  int h_stride, srs_I;
  float* slots;           // fp32 slot rows [S, H]
  int32_t* ctl;           // control words (kFusedCtlBytes)
  int spin_limit;         // polls before a wait gives up
  int hold;               // tests: the layout is never published, so every wait gives up
};
bool fused_fits(int wf, int T, int H, int E, int top_k, int I);
hipError_t launch_fused(int wf, const FusedArgs& a, hipStream_t st);

// finalize.hip
// combine: 1 fp32 slot rows, 2 fp32 token rows, 3 bf16 slot rows.
hipError_t launch_finalize(const void* out, int T, int H, int k1, int combine, uint16_t* y,
                           hipStream_t st);

}  // namespace mxmoe
