// C ABI of the MX MoE block: argument validation, workspace plan, launcher choice and the launch
// sequence route -> align -> quant -> gate_up (+SwiGLU, requant) -> down (+weighted combine) ->
// bf16 output. Everything is enqueued on the caller's stream; nothing is read back to the host.
#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include "mxmoe.h"
#include "device.h"
#include "kernels.h"

using namespace mxmoe;

namespace mxmoe {

namespace {
int env_int(const char* name, int unset) {
  const char* v = getenv(name);
  return v && *v ? atoi(v) : unset;
}
Tuning read_tuning() {
  Tuning t;
  t.trace = env_int("MXMOE_TRACE", 0) != 0;
  t.w_nt = env_int("MXMOE_W_NT", -1);
  t.xcd_order = env_int("MXMOE_XCD_ORDER", -1);
  t.xcd_run_gu = env_int("MXMOE_XCD_RUN_GU", -1);
  t.xcd_run_dn = env_int("MXMOE_XCD_RUN_DN", -1);
  t.stream_depth = env_int("MXMOE_STREAM_DEPTH", -1);
  t.prio = env_int("MXMOE_PRIO", -1);
  t.tile_pipe = env_int("MXMOE_TILE_PIPE", -1);
  t.slot_order = env_int("MXMOE_SLOT_ORDER", -1);
  t.cap_units = env_int("MXMOE_CAP_UNITS", -1);
  t.final_nt = env_int("MXMOE_NT", -1);
  t.gate_tile = env_int("MXMOE_GATE_TILE", -1);
  t.down_rows = env_int("MXMOE_DOWN_ROWS", -1);
  t.pair_fp4 = env_int("MXMOE_PAIR_FP4", -1);
  t.pf_steps = env_int("MXMOE_PF_STEPS", -1);
  t.pf_wgs = env_int("MXMOE_PF_WGS", -1);
  return t;
}
}  // namespace

const Tuning& tuning() {
  static const Tuning t = read_tuning();  // once per process
  return t;
}

}  // namespace mxmoe

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int wf_of(int w_fmt) {
  return w_fmt == MXMOE_MXFP8_E4M3 ? WF_FP8 : (w_fmt == MXMOE_MXFP4_E2M1 ? WF_FP4 : WF_BF16);
}

// Row size in bytes of the kernel-native scale layout for a K-long row.
int scale_row_bytes(int K) {
  int nks = (K + KSTEP - 1) / KSTEP;
  return 16 * ((nks + 3) / 4);
}

size_t cap_of(int S, int E1, int bm) {
  size_t cap = (size_t)S + (size_t)(E1 < S ? E1 : S) * (bm - 1);
  return (cap + bm - 1) / bm * bm;
}

// Largest batch whose final rounding runs inside the down pass: one wave per 64-column chunk
// converts all T rows of its chunk, so the tail grows with T.
constexpr int kFuseFinalMaxT = 256;

// Automatic launcher choice: block-major (large-M) tiles once the experts hold enough rows,
// measured by sweeping 32..4096 tokens through both launchers (forward time, cold weights):
//   hidden 3072, 128 experts, I 384 (MXFP8) or 768 (MXFP4), uniform or Zipf(1.1) routing: the
//     large-M launcher wins from S / (E+1) ~ 16 (16.5 uniform, ~16 Zipf) for both formats;
//   hidden 2048, 512 experts, I 512 (MXFP4): from ~16 with uniform routing, but from ~5.6 under
//     Zipf(1.1), where the popular experts hold ~T rows and the small-M launcher re-streams their
//     weights for every 16-row tile (512 tokens: 83 against 116 us).
// With many experts the threshold follows the skewed routing of that model family: a uniform
// 512-expert batch at 6..16 slots per expert runs 3-16% slower on the large-M launcher.
bool auto_large_m(int S, int E1) {
  const long long rows = (long long)S, e1 = E1;
  return E1 > 256 ? rows >= 6 * e1 : rows >= 16 * e1;
}

bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128 || bm == 256; }

int check_route_args(int T, int E, int top_k) {
  if (T < 0 || E < 1 || E > kMaxExperts || top_k < 1 || top_k > E) return MXMOE_EINVAL;
  if (top_k > kMaxTopK) return MXMOE_EUNSUPPORTED;
  if ((long long)T * (top_k + 1) > (1LL << 30)) return MXMOE_EUNSUPPORTED;
  return MXMOE_OK;
}

int check_shape(const mxmoe_shape* s) {
  if (!s) return MXMOE_EINVAL;
  int rc = check_route_args(s->T, s->E, s->top_k);
  if (rc) return rc;
  if (s->H <= 0 || s->I <= 0 || s->H % 32 || s->I % 32) return MXMOE_EINVAL;
  if (s->H % 128) return MXMOE_EUNSUPPORTED;
  if (s->logits_dtype != MXMOE_BF16 && s->logits_dtype != MXMOE_F32) return MXMOE_EINVAL;
  bool mxw = s->w_fmt == MXMOE_MXFP8_E4M3 || s->w_fmt == MXMOE_MXFP4_E2M1;
  if (!mxw && s->w_fmt != MXMOE_BF16) return MXMOE_EINVAL;
  // MX weights take MXFP8 activations; MXFP4 weights also MXFP4 activations (both MFMA operands
  // E2M1)
  if (mxw && s->act_fmt != MXMOE_MXFP8_E4M3 &&
      !(s->w_fmt == MXMOE_MXFP4_E2M1 && s->act_fmt == MXMOE_MXFP4_E2M1))
    return MXMOE_EUNSUPPORTED;
  if (!mxw && s->act_fmt != MXMOE_BF16) return MXMOE_EUNSUPPORTED;
  // one expert's prepacked W13 (W2 is half of it) is addressed with 32-bit offsets
  const double eb = s->w_fmt == MXMOE_MXFP8_E4M3 ? 1.0 : (s->w_fmt == MXMOE_MXFP4_E2M1 ? 0.5 : 2.0);
  if ((double)2 * s->I * s->H * eb >= (double)kMaxBufferBytes) return MXMOE_EUNSUPPORTED;
  return MXMOE_OK;
}

enum Seg {
  SEG_CTL, SEG_IDS, SEG_W, SEG_SORTED, SEG_BLOCKEXP, SEG_COUNTERS, SEG_EXPOFF, SEG_TOUCHED, SEG_ALIGN,
  SEG_XQ, SEG_XS, SEG_H, SEG_HS, SEG_OUT, SEG_DONE, SEG_SORTW, NSEG
};

struct Plan {
  int T, H, E, k, I, k1, S, E1;
  int wf;
  bool mx, large;
  int combine;  // 1 slots, 2 atomic, 3 bf16 slots
  bool fuse_final;  // final bf16 rounding inside the down pass (small M, atomic combine)
  int bm, cap, Ip, srs_H, srs_I;
  int xrow, hrow;  // bytes of an activation-code row [H] and of an intermediate row [Ip]
  int unit_run;  // large-M unit order from the options (0 = the launcher's default)
  bool fused;    // the one-launch path (small batches)
  bool so;       // slot-order plan: no sort (small-M launcher)
  int so_tiles;  // its shared-expert tiles of 16 tokens
  int hrows;     // intermediate rows: the layout's capacity, or T per expert in slot order
  int spin_limit, hold;
  size_t off[NSEG + 1];
};

// Every buffer the kernels address with 32-bit offsets stays below 2 GiB: activation codes and
// scales, the intermediate and its scales, and one expert's prepacked weights (the descriptors'
// range and the row offsets are 32-bit; the out-of-range sentinel 0x80000000 must not be valid).
bool within_offsets(const Plan& p) {
  const size_t lim = kMaxBufferBytes;
  if ((size_t)p.T * p.xrow >= lim) return false;
  if ((size_t)p.T * p.srs_H >= lim) return false;
  if ((size_t)p.hrows * p.hrow >= lim) return false;
  if ((size_t)p.hrows * p.srs_I >= lim) return false;
  return true;
}

int make_plan(const mxmoe_shape* s, const mxmoe_options* opt, Plan* P) {
  int rc = check_shape(s);
  if (rc) return rc;
  mxmoe_options o = opt ? *opt : mxmoe_options{0, 0, 0, 0, nullptr, 0, 0, 0, 0};
  if (o.launcher < 0 || o.launcher > 2 || o.combine < 0 || o.combine > 3 || o.unit_run < -1 ||
      o.fused < -1 || o.fused > 1 || o.spin_limit < 0 || o.hold < 0 || o.hold > 1 ||
      o.layout < 0 || o.layout > 2)
    return MXMOE_EINVAL;
  if (o.block_m != 0 && !valid_block_m(o.block_m)) return MXMOE_EINVAL;
  Plan& p = *P;
  p.T = s->T; p.H = s->H; p.E = s->E; p.k = s->top_k; p.I = s->I;
  p.k1 = p.k + 1; p.S = p.T * p.k1; p.E1 = p.E + 1;
  p.wf = wf_of(s->w_fmt);
  if (p.wf == WF_FP4 && s->act_fmt == MXMOE_MXFP4_E2M1) p.wf = WF_FP4A4;
  p.mx = p.wf != WF_BF16;
  p.large = o.launcher == MXMOE_LAUNCH_LARGE_M ||
            (o.launcher == MXMOE_LAUNCH_AUTO && auto_large_m(p.S, p.E1));
  // One launch for the whole block: small batches with the small-M plan (16-row tiles, fp32 slot
  // rows) whose layout fits the layout workgroup.
  const bool fused_ok = o.launcher != MXMOE_LAUNCH_LARGE_M &&
                        fused_fits(p.wf, p.T, p.H, p.E, p.k, p.I) &&
                        (o.combine == MXMOE_COMBINE_AUTO || o.combine == MXMOE_COMBINE_SLOTS) &&
                        (o.block_m == 0 || o.block_m == 16);
  if (o.fused == 1 && !fused_ok) return MXMOE_EUNSUPPORTED;
  p.fused = o.fused == 1 && fused_ok;
  if (p.fused) p.large = false;  // the one-launch path is a small-M plan
  p.spin_limit = o.spin_limit ? o.spin_limit : kFusedDefaultSpin;
  p.hold = o.hold;
  // Large batches write bf16 slot rows (fp32 atomics run at about one value per L2 channel per
  // cycle, far below what the prefill combine needs); small batches write fp32 slot rows. The
  // atomic combine at small M rounds to bf16 inside the down pass (no final launch), but waiting
  // for the atomics costs more than that launch at decode sizes (measured: 32 tokens, hidden
  // 3072: down 52 us against 36 us plus a 3 us final pass).
  p.combine = o.combine ? o.combine : (p.large ? MXMOE_COMBINE_SLOTS_BF16 : MXMOE_COMBINE_SLOTS);
  p.fuse_final = !p.large && p.combine == MXMOE_COMBINE_ATOMIC && p.T <= kFuseFinalMaxT;
  p.bm = o.block_m ? o.block_m : (p.large ? (p.mx ? 128 : 64) : 16);
  // Slot order (no sort; each small-M unit finds its expert's rows itself) where most experts
  // have rows and K is not split; requested explicitly, any small-M plan with 16-row tiles, slot
  // rows and at most kSlotOrderMaxT tokens.
  const bool so_ok = !p.large && !p.fused && p.combine != MXMOE_COMBINE_ATOMIC && p.bm == 16 &&
                     p.T <= kSlotOrderMaxT;
  if (o.layout == MXMOE_LAYOUT_SLOTS && !so_ok) return MXMOE_EUNSUPPORTED;
  p.so = o.layout == MXMOE_LAYOUT_SLOTS ||
         (o.layout == MXMOE_LAYOUT_AUTO && so_ok && tuning().slot_order != 0 &&
          slot_order_fits(p.T, p.E, p.k, p.I));
  p.so_tiles = (p.T + 15) / 16;
  p.cap = (int)cap_of(p.S, p.E1, p.bm);
  p.Ip = round_up(p.I, KSTEP);
  p.srs_H = scale_row_bytes(p.H);
  p.srs_I = scale_row_bytes(p.Ip);
  p.xrow = !p.mx ? 2 * p.H : (a_is_fp4(p.wf) ? p.H / 2 : p.H);
  p.hrow = !p.mx ? 2 * p.Ip : (a_is_fp4(p.wf) ? p.Ip / 2 : p.Ip);
  // slot order keeps T intermediate rows per expert (every expert's rows at a fixed place, so the
  // down pass needs no lookup before its copy); the automatic choice bounds what that costs
  if (p.so && o.layout == MXMOE_LAYOUT_AUTO &&
      (size_t)p.E1 * p.T * p.hrow > kSlotOrderMaxRowBytes)
    p.so = false;
  p.hrows = p.so ? std::max(p.cap, p.E1 * p.T) : p.cap;
  p.unit_run = o.unit_run;
  if (!within_offsets(p)) return MXMOE_EUNSUPPORTED;
  size_t sz[NSEG];
  sz[SEG_CTL] = kFusedCtlBytes;  // first in every plan, so any call may follow any other
  sz[SEG_IDS] = (size_t)p.S * 4;
  sz[SEG_W] = (size_t)p.S * 4;
  sz[SEG_SORTED] = (size_t)(p.so ? p.E1 * p.T : p.cap) * 4;  // slot order: per-expert slot lists
  sz[SEG_BLOCKEXP] = (size_t)(p.cap / p.bm) * 4;
  sz[SEG_COUNTERS] = 16;
  sz[SEG_EXPOFF] = (size_t)(p.E1 + 1) * 4;  // slot order: per-expert row counts
  sz[SEG_TOUCHED] = (size_t)p.E1 * 4;
  sz[SEG_ALIGN] = align_scratch_bytes(p.T, p.E, p.k);
  sz[SEG_XQ] = p.mx ? (size_t)p.T * p.xrow : 0;
  sz[SEG_XS] = p.mx ? (size_t)p.T * p.srs_H : 0;
  sz[SEG_H] = (size_t)p.hrows * p.hrow;
  sz[SEG_HS] = p.mx ? (size_t)p.hrows * p.srs_I : 0;
  sz[SEG_DONE] = p.fuse_final ? (size_t)(p.H / 64) * 4 : 0;
  sz[SEG_SORTW] = (size_t)p.cap * 4;
  sz[SEG_OUT] = p.combine == MXMOE_COMBINE_ATOMIC ? (size_t)p.T * p.H * 4
                                                  : (size_t)p.S * p.H * (p.combine == MXMOE_COMBINE_SLOTS ? 4 : 2);
  size_t at = 0;
  for (int i = 0; i < NSEG; ++i) {
    p.off[i] = at;
    at += up(sz[i]);
  }
  p.off[NSEG] = at;
  return MXMOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MXMOE_OK : MXMOE_EHIP; }

}  // namespace

extern "C" {

const char* mxmoe_status_string(int status) {
  switch (status) {
    case MXMOE_OK: return "ok";
    case MXMOE_EINVAL: return "invalid argument";
    case MXMOE_EUNSUPPORTED: return "unsupported shape or format";
    case MXMOE_EWORKSPACE: return "workspace too small or misaligned";
    case MXMOE_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int mxmoe_gate(const void* x, const void* w_gate, int T, int H, int E, int logits_dtype,
               void* logits, void* stream) {
  return mxmoe_gate_ex(x, w_gate, T, H, E, logits_dtype, 0, logits, stream);
}

int mxmoe_gate_ex(const void* x, const void* w_gate, int T, int H, int E, int logits_dtype,
                  int tile, void* logits, void* stream) {
  if (T < 0 || H <= 0 || H % 32 || E < 1 || E > kMaxExperts) return MXMOE_EINVAL;
  if (tile != 0 && !valid_gate_tile(tile)) return MXMOE_EINVAL;
  if ((size_t)T * H * 2 >= kMaxBufferBytes) return MXMOE_EUNSUPPORTED;
  if ((size_t)64 * H * 2 > 0x7FFFFFFFu) return MXMOE_EINVAL;  // tile offsets stay below 2^31
  if (logits_dtype != MXMOE_BF16 && logits_dtype != MXMOE_F32) return MXMOE_EINVAL;
  if (T == 0) return MXMOE_OK;
  if (!x || !w_gate || !logits) return MXMOE_EINVAL;
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(logits, logits_dtype == MXMOE_F32 ? 4 : 2))
    return MXMOE_EINVAL;
  return hip_status(launch_gate((const uint16_t*)x, (const uint16_t*)w_gate, T, H, E,
                                logits_dtype == MXMOE_F32, logits, tile, (hipStream_t)stream));
}

int mxmoe_route(const void* logits, int T, int E, int top_k, int logits_dtype, int32_t* topk_ids,
                float* topk_w, void* stream) {
  int rc = check_route_args(T, E, top_k);
  if (rc) return rc;
  if (logits_dtype != MXMOE_BF16 && logits_dtype != MXMOE_F32) return MXMOE_EINVAL;
  if (T == 0) return MXMOE_OK;
  if (!logits || !topk_ids || !topk_w) return MXMOE_EINVAL;
  if (!aligned(logits, logits_dtype == MXMOE_F32 ? 4 : 2) || !aligned(topk_ids, 4) ||
      !aligned(topk_w, 4))
    return MXMOE_EINVAL;
  return hip_status(launch_route(logits, logits_dtype == MXMOE_F32, T, E, top_k, topk_ids, topk_w,
                                 (hipStream_t)stream));
}

size_t mxmoe_align_capacity(int T, int E, int top_k, int block_m) {
  if (check_route_args(T, E, top_k) || !valid_block_m(block_m)) return 0;
  return cap_of(T * (top_k + 1), E + 1, block_m);
}

size_t mxmoe_align_workspace_bytes(int T, int E, int top_k, int block_m) {
  if (check_route_args(T, E, top_k) || !valid_block_m(block_m)) return 0;
  return align_scratch_bytes(T, E, top_k);
}

int mxmoe_align(const int32_t* topk_ids, int T, int E, int top_k, int block_m,
                int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_pad, void* stream) {
  return mxmoe_align_ex(topk_ids, T, E, top_k, block_m, sorted_ids, block_expert, num_post_pad,
                        nullptr, nullptr, 0, stream);
}

int mxmoe_align_ex(const int32_t* topk_ids, int T, int E, int top_k, int block_m,
                   int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_pad,
                   int32_t* expert_off, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_route_args(T, E, top_k);
  if (rc) return rc;
  if (!valid_block_m(block_m)) return MXMOE_EINVAL;
  if (T == 0) return MXMOE_OK;
  if (!topk_ids || !sorted_ids || !block_expert || !num_post_pad) return MXMOE_EINVAL;
  size_t need = align_scratch_bytes(T, E, top_k);
  if (need && (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)))
    return MXMOE_EWORKSPACE;
  AlignOut o{sorted_ids, block_expert, num_post_pad, expert_off, nullptr, nullptr, nullptr, nullptr};
  return hip_status(launch_align(topk_ids, T, E, top_k, block_m, o, workspace, (hipStream_t)stream));
}

int mxmoe_quantize(const void* src, int rows, int K, int src_dtype, int fmt, uint8_t* codes,
                   uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MXMOE_EINVAL;
  if (src_dtype != MXMOE_BF16 && src_dtype != MXMOE_F32) return MXMOE_EINVAL;
  if (fmt != MXMOE_MXFP8_E4M3 && fmt != MXMOE_MXFP4_E2M1) return MXMOE_EINVAL;
  if (rows == 0) return MXMOE_OK;
  if (!src || !codes || !scales) return MXMOE_EINVAL;
  if (!aligned(src, 16) || !aligned(codes, 16)) return MXMOE_EINVAL;
  return hip_status(launch_quantize_canonical(src, src_dtype == MXMOE_F32, rows, K,
                                              fmt == MXMOE_MXFP4_E2M1, codes, scales,
                                              (hipStream_t)stream));
}

static PrepackDims dims_of(const mxmoe_shape* s, bool w13) {
  PrepackDims d;
  d.E1 = s->E + 1;
  d.N = w13 ? 2 * s->I : s->H;
  d.K = w13 ? s->H : s->I;
  d.wf = wf_of(s->w_fmt);
  d.w13 = w13;
  d.I = s->I;
  return d;
}

size_t mxmoe_prepacked_bytes(const mxmoe_shape* s, int which) {
  if (check_shape(s) || which < 0 || which > 3) return 0;
  PrepackDims d = dims_of(s, which < 2);
  return (which & 1) ? prepack_scale_bytes(d) : prepack_code_bytes(d);
}

int mxmoe_prepack(const mxmoe_shape* s, const void* w13, const uint8_t* s13, const void* w2,
                  const uint8_t* s2, void* w13_p, void* s13_p, void* w2_p, void* s2_p,
                  void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  bool mx = s->w_fmt != MXMOE_BF16;
  if (!w13 || !w2 || !w13_p || !w2_p) return MXMOE_EINVAL;
  if (mx && (!s13 || !s2 || !s13_p || !s2_p)) return MXMOE_EINVAL;
  if (!aligned(w13, 16) || !aligned(w2, 16) || !aligned(w13_p, 16) || !aligned(w2_p, 16))
    return MXMOE_EINVAL;
  if (mx && (!aligned(s13_p, 4) || !aligned(s2_p, 4))) return MXMOE_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_prepack(dims_of(s, true), w13, s13, w13_p, s13_p, st);
  if (e == hipSuccess) e = launch_prepack(dims_of(s, false), w2, s2, w2_p, s2_p, st);
  return hip_status(e);
}

size_t mxmoe_workspace_bytes_ex(const mxmoe_shape* s, const mxmoe_options* opt) {
  Plan p;
  if (make_plan(s, opt, &p)) return 0;
  return p.off[NSEG];
}

size_t mxmoe_workspace_bytes(const mxmoe_shape* s) { return mxmoe_workspace_bytes_ex(s, nullptr); }

size_t mxmoe_workspace_view(const mxmoe_shape* s, const mxmoe_options* opt, int which,
                            size_t* bytes, int* block_m) {
  Plan p;
  if (make_plan(s, opt, &p)) return (size_t)-1;
  static const int segs[MXMOE_VIEW_COUNT] = {SEG_IDS, SEG_W,  SEG_SORTED, SEG_BLOCKEXP, SEG_COUNTERS,
                                             SEG_EXPOFF, SEG_XQ, SEG_XS, SEG_H, SEG_HS, SEG_CTL};
  if (which < 0 || which >= MXMOE_VIEW_COUNT) return (size_t)-1;
  const bool lay = !p.so;  // slot order: per-expert slot lists in place of the sorted rows
  const size_t sz[MXMOE_VIEW_COUNT] = {
      (size_t)p.S * 4, (size_t)p.S * 4, (size_t)(lay ? p.cap : p.E1 * p.T) * 4,
      lay ? (size_t)(p.cap / p.bm) * 4 : 0, lay ? 4u : 0u, lay ? (size_t)(p.E1 + 1) * 4 : 0, p.mx ? (size_t)p.T * p.xrow : 0, p.mx ? (size_t)p.T * p.srs_H : 0,
      (size_t)p.hrows * p.hrow, p.mx ? (size_t)p.hrows * p.srs_I : 0, 4};
  if (bytes) *bytes = sz[which];
  if (block_m) *block_m = p.bm;
  return p.off[segs[which]] + (which == MXMOE_VIEW_STATUS ? kFusedStatusByte : 0);
}

int mxmoe_forward_ex(const mxmoe_shape* s, const mxmoe_options* opt, const void* x,
                     const void* logits, const void* w13_p, const void* s13_p, const void* w2_p,
                     const void* s2_p, void* y, void* workspace, size_t workspace_bytes,
                     void* stream) {
  Plan P;
  int rc = make_plan(s, opt, &P);
  if (rc) return rc;
  if (P.T == 0) return MXMOE_OK;
  if (!x || !logits || !w13_p || !w2_p || !y) return MXMOE_EINVAL;
  if (P.mx && (!s13_p || !s2_p)) return MXMOE_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w13_p, 16) || !aligned(w2_p, 16) ||
      !aligned(logits, s->logits_dtype == MXMOE_F32 ? 4 : 2))
    return MXMOE_EINVAL;
  if (!workspace || workspace_bytes < P.off[NSEG] || !aligned(workspace, kAlign))
    return MXMOE_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  int32_t* ids = (int32_t*)(ws + P.off[SEG_IDS]);
  float* tw = (float*)(ws + P.off[SEG_W]);
  int32_t* sorted = (int32_t*)(ws + P.off[SEG_SORTED]);
  int32_t* bexp = (int32_t*)(ws + P.off[SEG_BLOCKEXP]);
  int32_t* counters = (int32_t*)(ws + P.off[SEG_COUNTERS]);  // [0] num_post_pad, [1] n_touched
  int32_t* eoff = (int32_t*)(ws + P.off[SEG_EXPOFF]);
  int32_t* touched = (int32_t*)(ws + P.off[SEG_TOUCHED]);
  void* aws = ws + P.off[SEG_ALIGN];
  uint8_t* xq = (uint8_t*)(ws + P.off[SEG_XQ]);
  uint8_t* xs = (uint8_t*)(ws + P.off[SEG_XS]);
  uint8_t* h = (uint8_t*)(ws + P.off[SEG_H]);
  uint8_t* hs = (uint8_t*)(ws + P.off[SEG_HS]);
  float* out32 = (float*)(ws + P.off[SEG_OUT]);
  int32_t* done = (int32_t*)(ws + P.off[SEG_DONE]);
  float* sorted_w = (float*)(ws + P.off[SEG_SORTW]);
  const bool slots = P.combine != MXMOE_COMBINE_ATOMIC;

  const Tuning& tn = tuning();
  if (tn.trace)
    fprintf(stderr, "mxmoe_forward: T=%d H=%d E=%d k=%d I=%d w=%d launcher=%s block_m=%d combine=%s\n",
            P.T, P.H, P.E, P.k, P.I, s->w_fmt,
            P.fused ? "one_launch" : (P.large ? "large_m" : (P.so ? "small_m_slot_order" : "small_m")), P.bm,
            P.combine == 1 ? "slots" : (P.combine == 2 ? "atomic" : "slots_bf16"));

  void** ev = opt ? opt->stage_events : nullptr;
  auto mark = [&](int i) -> hipError_t {
    return ev ? hipEventRecord((hipEvent_t)ev[i], st) : hipSuccess;
  };
  hipError_t e = mark(0);
  if (P.fused) {
    FusedArgs fa{};
    fa.x = (const uint16_t*)x;
    fa.logits = logits;
    fa.logits_f32 = s->logits_dtype == MXMOE_F32;
    fa.w13 = (const uint8_t*)w13_p;
    fa.s13 = (const uint8_t*)s13_p;
    fa.w2 = (const uint8_t*)w2_p;
    fa.s2 = (const uint8_t*)s2_p;
    fa.y = (uint16_t*)y;
    fa.T = P.T; fa.H = P.H; fa.E = P.E; fa.top_k = P.k; fa.I = P.I; fa.Ip = P.Ip;
    fa.ids = ids;
    fa.tw = tw;
    fa.lay = AlignOut{sorted, bexp, counters, eoff, touched, counters + 1, tw, sorted_w};
    fa.cap = P.cap;
    fa.xq = xq;
    fa.xs = xs;
    fa.srs_H = P.srs_H;
    fa.h = h;
    fa.hs = hs;
    fa.h_stride = P.Ip;
    fa.srs_I = P.srs_I;
    fa.slots = out32;
    fa.ctl = (int32_t*)(ws + P.off[SEG_CTL]);
    fa.spin_limit = P.spin_limit;
    fa.hold = P.hold;
    if (e == hipSuccess) e = launch_fused(P.wf, fa, st);
    for (int i = 1; i < MXMOE_STAGE_EVENTS && e == hipSuccess; ++i) e = mark(i);
    return hip_status(e);
  }
  PrologueArgs pa;
  pa.logits = logits;
  pa.T = P.T;
  pa.E = P.E;
  pa.top_k = P.k;
  pa.ids = ids;
  pa.w = tw;
  pa.block_m = P.bm;
  pa.cap = P.cap;
  pa.out = AlignOut{sorted, bexp, counters, eoff, touched, counters + 1, tw, sorted_w};
  pa.x = (const uint16_t*)x;
  pa.H = P.H;
  pa.xq = P.mx ? xq : nullptr;
  pa.xs = xs;
  pa.a4 = a_is_fp4(P.wf);
  pa.srs = P.srs_H;
  pa.zero_out = slots ? nullptr : out32;
  pa.zero_cnt = P.fuse_final ? done : nullptr;
  pa.n_cnt = P.fuse_final ? P.H / 64 : 0;
  pa.no_sort = P.so;
  pa.pf_w = nullptr;
  {
    // slot-order gate_up: its units' first weight K-steps go into each XCD's L2 while the routing
    // runs (the units' mapping onto XCDs is that of k_gemm_stream's per-XCD ranges)
    const int pf_steps = tn.pf_steps >= 0 ? tn.pf_steps : kPrefetchSteps;
    const int nks = P.H / KSTEP;
    const bool ranges = tn.xcd_order != 0;
    if (P.so && P.wf == WF_FP8 && ranges && pf_steps > 0 && pf_steps <= nks) {
      const int fb = 2048;  // bytes of an fp8 weight fragment
      pa.pf_w = (const uint8_t*)w13_p;
      pa.pf_ws = (const uint8_t*)s13_p;
      pa.pf_wbytes = (size_t)(2 * P.I / 16) * nks * fb;
      pa.pf_sbytes = (size_t)(2 * P.I / 64) * nks * 256;
      pa.pf_chunks = P.I / 32;
      pa.pf_nb = P.E + P.so_tiles;
      pa.pf_nks = nks;
      pa.pf_step_bytes = 4 * fb;
      pa.pf_steps = pf_steps;
      pa.pf_wgs = tn.pf_wgs > 0 ? tn.pf_wgs : kPrefetchWgs;
    }
  }
  if (e == hipSuccess) e = launch_prologue(pa, s->logits_dtype == MXMOE_F32, aws, st);
  const int n_blocks = P.cap / P.bm;
  GemmParams g{};
  g.sorted_ids = sorted;
  g.expert_off = eoff;
  g.touched = touched;
  g.n_touched = counters + 1;
  g.block_expert = bexp;
  g.num_post_pad = counters;
  g.block_m = P.bm;
  g.S = P.S;
  g.k1 = P.k1;
  g.I = P.I;
  g.Ip = P.Ip;
  g.H = P.H;
  g.h = h;
  g.hs = hs;
  g.h_stride = P.hrow;
  g.h_srs = P.srs_I;
  g.topk_w = tw;
  g.sorted_w = sorted_w;
  g.out32 = out32;
  g.combine = P.combine;
  g.T = P.T;
  g.so = P.so;
  g.so_tiles = P.so_tiles;
  g.so_cap = P.T;
  // an expert is without rows with probability about exp(-T k / E): below ~5% the down pass issues
  // its weights before it reads the count
  g.so_spec = (long)P.T * P.k > 3L * P.E;
  g.E = P.E;
  g.topk_ids = ids;
  g.so_list = sorted;
  g.so_cnt = eoff;
  g.xcd_order = tn.xcd_order >= 0 ? tn.xcd_order != 0 : 1;
  g.w_nt = tn.w_nt >= 0 ? tn.w_nt != 0 : 1;
  // large-M unit order: the options' run (-1: one contiguous range per XCD), else the A/B switch,
  // else (-1 here) the launcher's own default
  auto unit_run = [&](int deflt, int env) { return P.unit_run ? (P.unit_run < 0 ? 0 : P.unit_run)
                                                              : (env >= 0 ? env : deflt); };
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess) {
    GemmParams gu = g;
    gu.a = P.mx ? xq : (const uint8_t*)x;
    gu.as = xs;
    gu.a_stride = P.xrow;
    gu.a_srs = P.srs_H;
    gu.a_bytes = (uint32_t)((size_t)P.T * gu.a_stride);
    gu.as_bytes = (uint32_t)((size_t)P.T * P.srs_H);
    gu.w = (const uint8_t*)w13_p;
    gu.ws = (const uint8_t*)s13_p;
    gu.NT = 2 * P.I / 16;
    gu.NKS = P.H / KSTEP;
    gu.xcd_run = unit_run(-1, tn.xcd_run_gu);
    e = launch_gate_up(P.wf, P.large, gu, n_blocks, st);
  }
  if (e == hipSuccess) e = mark(2);
  if (e == hipSuccess) {
    GemmParams dn = g;
    dn.a = h;
    dn.as = hs;
    dn.a_stride = g.h_stride;
    dn.a_srs = P.srs_I;
    dn.a_bytes = (uint32_t)((size_t)P.hrows * dn.a_stride);
    dn.as_bytes = (uint32_t)((size_t)P.hrows * P.srs_I);
    dn.w = (const uint8_t*)w2_p;
    dn.ws = (const uint8_t*)s2_p;
    dn.xcd_run = unit_run(-1, tn.xcd_run_dn);
    dn.NT = P.H / 16;
    dn.NKS = P.Ip / KSTEP;
    if (P.fuse_final) {
      dn.y = (uint16_t*)y;
      dn.chunk_done = done;
    }
    e = launch_down(P.wf, P.large, dn, n_blocks, st);
  }
  if (e == hipSuccess) e = mark(3);
  if (e == hipSuccess && !P.fuse_final)
    e = launch_finalize(out32, P.T, P.H, P.k1, P.combine, (uint16_t*)y, st);
  if (e == hipSuccess) e = mark(4);
  return hip_status(e);
}

int mxmoe_forward(const mxmoe_shape* s, const void* x, const void* logits, const void* w13_p,
                  const void* s13_p, const void* w2_p, const void* s2_p, void* y,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return mxmoe_forward_ex(s, nullptr, x, logits, w13_p, s13_p, w2_p, s2_p, y, workspace,
                          workspace_bytes, stream);
}

}  // extern "C"
