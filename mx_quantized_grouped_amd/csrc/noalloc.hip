// mxmoe_forward_noalloc: the whole block with its workspace in a device-resident array of the
// library instead of caller-provided memory, for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope __device__ array: every GPU the library runs on holds its own copy
// for the life of the process, at its own device address. In host code the name `scratch` is
// only a host-side stand-in for the symbol, never a device address, so host code never passes it
// anywhere: the device address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept in `g_scratch`; kernels receive that pointer as their workspace
// argument, exactly as they receive a caller's workspace in mxmoe_forward. At the same set-up the
// array's control words are cleared once, as mxmoe_forward requires of a new workspace.
#include <mutex>

#include "mxmoe.h"
#include "kernels.h"

static __device__ __align__(256) uint8_t scratch[MXMOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// Device address of this device's `scratch`, looked up on the first call per device.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXMOE_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXMOE_EHIP;
    // the workspace's control words start at zero (every forward call leaves them zero)
    if (hipMemset(p, 0, MXMOE_WORKSPACE_CONTROL_BYTES) != hipSuccess) return MXMOE_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MXMOE_OK;
}

}  // namespace

extern "C" int mxmoe_forward_noalloc(const mxmoe_shape* s, const void* x, const void* logits,
                                     const void* w13_p, const void* s13_p, const void* w2_p,
                                     const void* s2_p, void* y, void* stream) {
  // Every argument is checked before the first HIP call: the shape (an invalid one makes the
  // workspace size 0, and forward then returns its status without touching the GPU), T = 0, the
  // pointers and their alignment, then the size limit of the array.
  const size_t need = mxmoe_workspace_bytes(s);
  if (need == 0) return mxmoe_forward(s, x, logits, w13_p, s13_p, w2_p, s2_p, y, nullptr, 0, stream);
  if (s->T == 0) return MXMOE_OK;
  auto aligned = [](const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; };
  const bool mx = s->w_fmt != MXMOE_BF16;
  if (!x || !logits || !w13_p || !w2_p || !y || (mx && (!s13_p || !s2_p))) return MXMOE_EINVAL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w13_p, 16) || !aligned(w2_p, 16) ||
      !aligned(logits, s->logits_dtype == MXMOE_F32 ? 4 : 2))
    return MXMOE_EINVAL;
  if (need > (size_t)MXMOE_NOALLOC_SCRATCH_BYTES) return MXMOE_EWORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc != MXMOE_OK) return rc;
  return mxmoe_forward(s, x, logits, w13_p, s13_p, w2_p, s2_p, y, ws,
                       (size_t)MXMOE_NOALLOC_SCRATCH_BYTES, stream);
}
