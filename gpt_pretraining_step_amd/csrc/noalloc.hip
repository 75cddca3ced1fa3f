// The attention backward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): gpt2_op_attention_bwd_noalloc runs the same kernels as
// gpt2_op_attention_bwd, with its per-row buffers (D = rowsum(dO o O) and
// the log-sum-exp in log2 units, the workspace of gpt2_op_attention_bwd) in a
// static device array of this library instead of a caller-given workspace.
//
// The array lives on every GPU the library runs on until the process ends.
// Host code never uses its name as an address: on each device, the first
// call (with that device current) asks the runtime for the device address of
// the array and keeps it for that device.  Every call on one GPU shares that
// GPU's array; the kernels write every entry they read, so nothing needs
// clearing between calls, but calls that overlap in time on one GPU (two
// streams, two threads) race on it.
#include <mutex>

#include "common.h"

constexpr size_t kNoAllocFloats = size_t(1) << 21;  // 8 MiB: two floats per row, B * H * T <= 1,048,576

static __device__ __align__(256) float scratch[kNoAllocFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch` (nullptr on failure).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t gpt2_noalloc_scratch_bytes(void) { return kNoAllocFloats * sizeof(float); }

int gpt2_op_attention_bwd_noalloc(void* stream, int dtype, int B, int T, int H, int Hkv, int hd, const void* d_qkv,
                                  const void* d_y, const void* d_dy, const float* d_lse, void* d_dqkv,
                                  const int32_t* d_seg, const float* d_rope) {
  if (!d_qkv || !d_y || !d_dy || !d_lse || !d_dqkv) return GPT2_ERR_ARG;
  if (B < 1 || T < 1 || H < 1 || Hkv < 1 || H % Hkv) return GPT2_ERR_SHAPE;
  if (dtype == GPT2_PRECISION_BF16 ? hd != 64 : (dtype != GPT2_PRECISION_FP32 || hd < 1 || hd > 64))
    return GPT2_ERR_SHAPE;
  if (g2::attention_bwd_scratch(B, T, H) > kNoAllocFloats * sizeof(float)) return GPT2_ERR_SHAPE;
  if (d_rope && (dtype != GPT2_PRECISION_BF16 || ((uintptr_t)d_rope & 15))) return GPT2_ERR_ARG;
  void* ws = scratch_ptr();
  if (!ws) return GPT2_ERR_HIP;
  const hipError_t e = g2::launch_attention_bwd(g2::Launch{static_cast<hipStream_t>(stream), nullptr, ""}, dtype, B,
                                                T, H, Hkv, hd, d_qkv, d_y, d_dy, d_lse, d_dqkv, ws, d_seg,
                                                reinterpret_cast<const float2*>(d_rope));
  return e == hipSuccess ? GPT2_OK : GPT2_ERR_HIP;
}

}  // extern "C"
