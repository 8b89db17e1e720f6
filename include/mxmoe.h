/* mxmoe.h — C ABI of the MX-quantised sparse MoE expert block for AMD Instinct MI355X (gfx950).
 *
 * The block (per token t, bf16 activations x[t] of width H, bf16 router logits over E experts):
 *   route   top-k experts by logit, softmax weights over the k selected, and the shared expert
 *           (id E) appended as an always-selected slot with weight 1. The shared expert folded into
 *           the routing table is the change described in "Lần theo điểm nghẽn: Tối ưu MiniMax M3 trên
 *           AMD Instinct MI355X" (shared-expert passage, Fig. 4).
 *   align   counting sort of the T*(k+1) slots into expert-contiguous, tile-padded blocks (the work
 *           list of the grouped GEMMs; same page, local-shapes passage on grouped MoE programs).
 *   quant   x -> MXFP8 (E4M3 codes, one E8M0 scale per 32 along H), once per token.
 *   gate_up grouped GEMM over the routed + shared experts on gfx950 block-scaled MFMA, SwiGLU
 *           (SiLU(gate) * up) epilogue, requantised to MXFP8 along I.
 *   down    grouped GEMM, then the top-k weighted combine back to token order ("finalize", fused
 *           into the GEMM epilogue as in "Tối ưu hiệu năng Kimi K3 trong vLLM", deferred-finalize
 *           passage), and one rounding to bf16.
 * Weights are MXFP8 (E4M3) or MXFP4 (E2M1) with 32-element blocks and E8M0 scales along K, or
 * plain bf16. Encodings follow the OCP Microscaling Formats (MX) v1.0 specification.
 *
 * Conventions for every entry point:
 *   - Pointers are device memory owned by the caller unless a comment says "host". The library
 *     never allocates, frees, aborts, throws or exits.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is enqueued on it
 *     and the call returns without synchronising; nothing crosses back to the host (counts stay on
 *     the GPU, as the batch-1 decode page "Ling-3.0-flash: Tối ưu hóa độ trễ giải mã lên 54% trên
 *     4 GPU Blackwell" requires in "Hình dạng của một bước batch-1"), so calls are capturable.
 *   - Arguments are validated on the host before any HIP call; a failure returns a negative status
 *     and enqueues nothing. A launch failure returns MXMOE_EHIP. Faults inside a kernel surface at
 *     the caller's next synchronisation. T = 0 is a no-op returning MXMOE_OK.
 *   - Inputs must be finite (NaN/Inf logits or activations are a precondition violation).
 *   - Concurrent calls need distinct outputs and workspaces.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------------------------- status */
enum {
  MXMOE_OK = 0,
  MXMOE_EINVAL = -1,       /* null pointer, bad size, bad shape */
  MXMOE_EUNSUPPORTED = -2, /* valid but not implemented (format pair, shape class) */
  MXMOE_EWORKSPACE = -3,   /* workspace too small or misaligned */
  MXMOE_EHIP = -4          /* a HIP launch failed */
};

/* Data formats. */
enum {
  MXMOE_BF16 = 0,
  MXMOE_F32 = 1,
  MXMOE_MXFP8_E4M3 = 2, /* one code per byte */
  MXMOE_MXFP4_E2M1 = 3  /* two codes per byte: element 2i in the low nibble, 2i+1 in the high */
};

/* Launcher choice (small-M = expert-major decode grid, large-M = block-major prefill grid). */
enum { MXMOE_LAUNCH_AUTO = 0, MXMOE_LAUNCH_SMALL_M = 1, MXMOE_LAUNCH_LARGE_M = 2 };
/* Combine of the k+1 slot outputs of a token: per-slot fp32 rows summed in a fixed order
   (deterministic), fp32 atomics into a token-major accumulator (order varies run to run), or
   per-slot rows rounded to bf16 and summed in a fixed order (half the traffic of fp32 rows; one
   extra rounding per slot). */
enum { MXMOE_COMBINE_AUTO = 0, MXMOE_COMBINE_SLOTS = 1, MXMOE_COMBINE_ATOMIC = 2,
       MXMOE_COMBINE_SLOTS_BF16 = 3 };

/* Problem shape. Requirements: T >= 0; H % 128 == 0; I % 32 == 0; 1 <= top_k <= E <= 1024;
   w_fmt in {BF16, MXFP8_E4M3, MXFP4_E2M1}; act_fmt = BF16 for bf16 weights, MXFP8_E4M3 for MX
   weights, or MXFP4_E2M1 with MXFP4_E2M1 weights (W4A4: the activations and the SwiGLU
   intermediate are quantised to MXFP4 and both MFMA operands are E2M1); logits_dtype in
   {BF16, F32}. The kernels address each of these with 32-bit offsets, so each must stay below
   2 GiB, or the call returns MXMOE_EUNSUPPORTED: one expert's W13 codes, the activation codes
   (T*H bytes; T*H/2 for MXFP4, 2*T*H for bf16) and the intermediate (about T*(top_k+1)*I bytes
   plus tile padding; half that for MXFP4, twice for bf16). */
typedef struct {
  int32_t T, H, E, top_k, I;
  int32_t w_fmt, act_fmt, logits_dtype;
} mxmoe_shape;

/* Optional knobs for A/B runs, tests and timing; all-zero = automatic. */
typedef struct {
  int32_t launcher; /* MXMOE_LAUNCH_* */
  int32_t combine;  /* MXMOE_COMBINE_* */
  int32_t block_m;  /* align tile height (16, 32, 64, 128, 256); 0 = the launcher's default */
  /* Large-M unit order over the 8 XCDs (workgroups go round-robin over them): each XCD takes runs
     of unit_run consecutive output tiles in turn. 0 = the launcher's default (runs of 4 row
     tiles with all their column chunks), -1 = one contiguous range per XCD, 1 = plain linear
     order. Only which workgroup computes which tile changes: outputs are bit-identical. */
  int32_t unit_run;
  /* Optional array of MXMOE_STAGE_EVENTS caller-created hipEvent_t (passed as void*), recorded on
     the stream at the stage boundaries of mxmoe_forward_ex: before the prologue (routing, sort and
     activation quantisation), before gate_up, before down, before the final bf16 rounding, and
     after it. NULL = no events. */
  void** stage_events;
  /* The whole block in one launch for small batches (routing, layout, gate_up, down and the final
     sum as roles of one grid; small-M plan with 16-row tiles and fp32 slot rows; MX weights with
     MXFP8 activations, up to 128 tokens): 0 = the library's choice, 1 = required
     (MXMOE_EUNSUPPORTED if the shape or the other options do not allow it), -1 = never. */
  int32_t fused;
  /* One-launch path: polls of a bounded wait before it gives up (0 = the default, about 50 ms).
     A wait that gives up skips the work that depended on it, every workgroup still ends, and the
     status word (workspace view MXMOE_VIEW_STATUS) reads 1 after the call. */
  int32_t spin_limit;
  int32_t hold;     /* tests only: 1 = the one-launch path never publishes its layout, so every
                       wait on it gives up (exercises the bounded waits); 0 otherwise */
  /* Row layout of the small-M launcher, MXMOE_LAYOUT_*: AUTO = the library's choice; SORTED = the
     aligned layout of mxmoe_align (slots sorted by expert, tiles padded to block_m); SLOTS = no
     sort: every expert owns T rows of the intermediate, the gate_up units find a routed expert's
     slots themselves by a scan of the routing table (in slot order; the shared expert's are its
     tokens in order) and record them for the down pass. SLOTS needs the small-M launcher,
     16-row tiles, a slot-row combine and T <= 256 (MXMOE_EUNSUPPORTED otherwise); AUTO takes it
     where at least as many slots as experts make most experts' scans find rows and the
     intermediate of T rows per expert stays within 64 MiB. Each output row is the same sums in
     the same order in both layouts (bit-identical outputs), except where the sorted plan splits
     K over four waves (few units: a handful of tokens), which reorders the sums. */
  int32_t layout;
} mxmoe_options;
enum { MXMOE_LAYOUT_AUTO = 0, MXMOE_LAYOUT_SORTED = 1, MXMOE_LAYOUT_SLOTS = 2 };
#define MXMOE_STAGE_EVENTS 5

/* Host: static description of a status code. Never NULL. */
const char* mxmoe_status_string(int status);

/* ---------------------------------------------------------------------------------- gate
 * Router gate, the step in front of route: logits[t, e] = sum_h x[t, h] * w_gate[e, h] with bf16
 * operands and fp32 accumulation (the bf16 gate of "Ling-3.0-flash: Tối ưu hóa độ trễ giải mã lên
 * 54% trên 4 GPU Blackwell", section "Sửa thước đo trước khi sửa máy").
 * x      [T, H] bf16 row-major, 16-byte aligned; H % 32 == 0.
 * w_gate [E, H] bf16 row-major, 16-byte aligned; 1 <= E <= the routed-expert limit.
 * logits [T, E] row-major, written as fp32 (logits_dtype MXMOE_F32) or bf16 rounded to nearest
 *        even (MXMOE_BF16); its dtype is what mxmoe_route / mxmoe_forward then take.
 * The sum over h is split and combined in a fixed order: results are reproducible run to run.
 * T == 0 is a no-op. Bad sizes, null pointers or misalignment return MXMOE_EINVAL before any
 * HIP call; the caller owns every buffer. */
int mxmoe_gate(const void* x, const void* w_gate, int T, int H, int E, int logits_dtype,
               void* logits, void* stream);
/* mxmoe_gate with an explicit tile (for tests and A/B runs): 0 = chosen by shape; register tiles
 * 10*TM + F (TM 16-row token groups per wave, F 16-column expert groups: 11, 12, 14, 21, 22, 24,
 * 28, 41, 42, 44, 48, 84) or LDS-staged tiles 100 + 10*TM + F (124, 142, 144, 148). Every tile
 * splits the sum over H the same way, so the logits are bit-identical whatever the tile; another
 * value returns MXMOE_EINVAL. */
int mxmoe_gate_ex(const void* x, const void* w_gate, int T, int H, int E, int logits_dtype,
                  int tile, void* logits, void* stream);

/* --------------------------------------------------------------------------------- route
 * Top-k routing with the fixed lowest-index tie-break.
 * logits   [T, E] row-major, bf16 or fp32 (logits_dtype).
 * topk_ids [T, top_k+1] int32: for each token the top_k experts ordered by (logit descending,
 *          expert index ascending), -0 equal to +0; slot top_k holds the shared expert id E.
 * topk_w   [T, top_k+1] fp32: exp(l_j - l_0) / sum_{i<top_k} exp(l_i - l_0) for j < top_k
 *          (softmax renormalised over the selected experts); slot top_k holds exactly 1.0.
 * Selection compares logits, not probabilities (softmax is monotone; the MiniMax-M3 page's
 * speculative-indexer passage: a positive rescale cannot change a top-k order). */
int mxmoe_route(const void* logits, int T, int E, int top_k, int logits_dtype,
                int32_t* topk_ids, float* topk_w, void* stream);

/* --------------------------------------------------------------------------------- align
 * Counting sort of the flat slots f = t*(top_k+1) + j (S = T*(top_k+1) of them) by expert.
 * Experts 0..E (shared last) in ascending id order; within an expert ascending f (stable); each
 * expert's run is padded with the sentinel S to a multiple of block_m; experts with no slot get no
 * block. Outputs (sizes from mxmoe_align_capacity, cap = elements of sorted_ids):
 *   sorted_ids   [cap]          slot ids, S in padding and past the end
 *   block_expert [cap/block_m]  expert of each tile, -1 past the last used tile
 *   num_post_pad [1]            padded slot count in use
 *   expert_off   [E+2]          start of each expert's run (expert_off[E+1] = num_post_pad); may
 *                               be NULL
 * workspace: mxmoe_align_workspace_bytes(...) bytes of device scratch (may be 0 / NULL when that
 * returns 0). block_m in {16, 32, 64, 128, 256}. */
size_t mxmoe_align_capacity(int T, int E, int top_k, int block_m);       /* host; 0 if invalid */
size_t mxmoe_align_workspace_bytes(int T, int E, int top_k, int block_m); /* host */
int mxmoe_align_ex(const int32_t* topk_ids, int T, int E, int top_k, int block_m,
                   int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_pad,
                   int32_t* expert_off, void* workspace, size_t workspace_bytes, void* stream);
/* The same sort without expert offsets or workspace: the library allocates nothing, so this form
 * takes only sorts that need no scratch (those mxmoe_align_workspace_bytes sizes at 0: at most
 * 4096 slots) and returns MXMOE_EWORKSPACE for larger ones (use mxmoe_align_ex). */
int mxmoe_align(const int32_t* topk_ids, int T, int E, int top_k, int block_m,
                int32_t* sorted_ids, int32_t* block_expert, int32_t* num_post_pad, void* stream);

/* ------------------------------------------------------------------------------ quantize
 * MX quantisation of a row-major matrix src [rows, K] (bf16 or fp32, finite) along K, one scale
 * per 32 elements: shared_exp = floor(log2(max|x|)) - emax (8 for E4M3, 2 for E2M1) clamped to
 * [-127, 127]; scale byte = shared_exp + 127 (0 for an all-zero block); each element rounded to
 * the nearest code of x / 2^shared_exp, ties to even, saturating (448 / 6), sign kept.
 * codes  [rows, K] (MXFP8) or [rows, K/2] (MXFP4, low nibble first); scales [rows, K/32].
 * K % 32 == 0. The same rule quantises activations inside mxmoe_forward; this entry point is for
 * weights at load time. */
int mxmoe_quantize(const void* src, int rows, int K, int src_dtype, int fmt, uint8_t* codes,
                   uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------------- prepack
 * Converts canonical expert weights into the kernel-native, fragment-major layout, once at load
 * (the MiniMax-M3 page, shared-expert passage: weight and scale reordering moved to model load;
 * the serving loop uses the prepared form directly).
 * Canonical layouts (row-major, K contiguous; expert E is the shared expert):
 *   w13 [E+1, 2I, H] codes (gate rows 0..I-1, then up rows I..2I-1), s13 [E+1, 2I, H/32]
 *   w2  [E+1, H, I]  codes,                                            s2  [E+1, H, I/32]
 * Codes are bf16 values for BF16 weights (s13/s2 then NULL), one byte per code for MXFP8, two per
 * byte (low nibble first) for MXFP4. Output buffer sizes: mxmoe_prepacked_bytes(s, which) with
 * which = 0 (w13_p), 1 (s13_p), 2 (w2_p), 3 (s2_p); 0 for the scale buffers of BF16 weights. */
size_t mxmoe_prepacked_bytes(const mxmoe_shape* s, int which);
int mxmoe_prepack(const mxmoe_shape* s, const void* w13, const uint8_t* s13, const void* w2,
                  const uint8_t* s2, void* w13_p, void* s13_p, void* w2_p, void* s2_p,
                  void* stream);

/* ------------------------------------------------------------------------------- forward
 * The whole block. x [T, H] bf16; logits [T, E] (logits_dtype); prepacked weights from
 * mxmoe_prepack; y [T, H] bf16, overwritten. workspace: device scratch of at least
 * mxmoe_workspace_bytes(s) (or _ex with the same options), 256-byte aligned. Its first
 * MXMOE_WORKSPACE_CONTROL_BYTES bytes are the control words of the one-launch path: they must be
 * zero before the workspace's first forward call (allocate it zeroed or clear it once), and every
 * call leaves them zero again, also a call whose waits gave up. The rest of the workspace needs no
 * initialisation and is clobbered. */
#define MXMOE_WORKSPACE_CONTROL_BYTES (72u * 1024u)
size_t mxmoe_workspace_bytes(const mxmoe_shape* s);
size_t mxmoe_workspace_bytes_ex(const mxmoe_shape* s, const mxmoe_options* opt);
int mxmoe_forward(const mxmoe_shape* s, const void* x, const void* logits, const void* w13_p,
                  const void* s13_p, const void* w2_p, const void* s2_p, void* y,
                  void* workspace, size_t workspace_bytes, void* stream);
int mxmoe_forward_ex(const mxmoe_shape* s, const mxmoe_options* opt, const void* x,
                     const void* logits, const void* w13_p, const void* s13_p, const void* w2_p,
                     const void* s2_p, void* y, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------------------------ forward, no allocation
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): mxmoe_forward with the automatic plan, its workspace
 * being a device-resident array inside the library of MXMOE_NOALLOC_SCRATCH_BYTES per GPU (each
 * GPU the library runs on holds it until the process ends). The caller passes inputs, weights
 * and the output as for mxmoe_forward; the stream must belong to the current device. The call
 * allocates and frees nothing. A shape whose workspace (mxmoe_workspace_bytes) exceeds the array
 * returns MXMOE_EWORKSPACE before any HIP call. Every call on one GPU uses the same array and
 * leaves its contents behind; forward needs no initialised workspace, so nothing is cleared, but
 * calls that overlap on one GPU (other streams, other host threads) race on the array and must
 * be serialised by the caller. */
#define MXMOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int mxmoe_forward_noalloc(const mxmoe_shape* s, const void* x, const void* logits,
                          const void* w13_p, const void* s13_p, const void* w2_p, const void* s2_p,
                          void* y, void* stream);

/* Host: where forward keeps an intermediate inside its workspace, for inspection after the call
 * (routing table, sorted layout, quantised activations, quantised SwiGLU output). which:
 * 0 topk_ids, 1 topk_w, 2 sorted_ids, 3 block_expert, 4 num_post_pad, 5 expert_off,
 * 6 activation codes [T, H] (E4M3, MX weights only; size 0 otherwise), 7 activation scale bytes
 * [T, srs] with srs = H/32 rounded up to a multiple of 16 (K-block order, padding bytes
 * unspecified), 8 intermediate rows [cap, Ip] in the sorted layout's row order (row r belongs to
 * slot sorted_ids[r]; Ip = I rounded up to a multiple of 128; E4M3 codes for MX weights, bf16
 * values for bf16 weights), 9 intermediate scale bytes [cap, srs_I] (K-block order, srs_I = Ip/32
 * rounded up to a multiple of 16; MX weights only). Rows of padding slots and columns past I are
 * unspecified. In the slot-order plan (mxmoe_options.layout) view 2 holds (E+1)*T entries, entry
 * e*T + i the slot of expert e's i-th row (slot order; T*(top_k+1) past its count), views 3-5
 * have size 0, and row e*T + i of views 8 and 9 belongs to entry e*T + i of view 2.
 * 10 (MXMOE_VIEW_STATUS) the status word of the last one-launch call on this
 * workspace (int32: 0 every wait completed, 1 a bounded wait gave up and the output is not valid).
 * Returns the byte offset and writes the byte size to *bytes; the tile height forward used is
 * written to *block_m. Returns (size_t)-1 for an invalid request. */
#define MXMOE_VIEW_STATUS 10
#define MXMOE_VIEW_COUNT 11
size_t mxmoe_workspace_view(const mxmoe_shape* s, const mxmoe_options* opt, int which,
                            size_t* bytes, int* block_m);

#ifdef __cplusplus
}
#endif
#endif /* MXMOE_H */
