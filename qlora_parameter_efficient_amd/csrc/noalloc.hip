// Backward of the adapted linear layer for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc): lq_lora_bwd with its workspace in a static device
// array instead of a caller buffer.
//
// The array is a file-scope __device__ object, so each GPU the library runs
// on holds its own copy, at its own address, from module load until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the first call on a device asks
// the runtime for that device's address once and keeps it.  Calls on one GPU
// share the array; the backward's kernels clear what must start at zero (the
// split-K flags) themselves on every call, and every other
// part of the workspace is written before it is read, so stale contents from
// an earlier call do no harm.  Calls that overlap in time on one GPU race.
#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = LQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// this device's address of `scratch`, looked up once per device (the
// device current at the call is the one the stream belongs to)
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return lq::hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) {
    lq::set_error("device %d outside the %d devices the static workspace covers", dev,
                  kMaxDevices);
    return LQ_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return lq::hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) {
      lq::set_error("hipGetSymbolAddress(scratch) returned NULL");
      return LQ_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LQ_OK;
}

}  // namespace

extern "C" int lq_lora_bwd_noalloc(const void* dY, const void* X, int64_t M, const lq_weight* W0,
                                   const void* A, const void* B, int64_t r, float scale,
                                   lq_dtype dt, const float* T_saved, void* dX, float* dA,
                                   float* dB, int32_t accumulate, hipStream_t stream) {
  if (!W0) {
    lq::set_error("W0 descriptor is NULL");
    return LQ_ERR_INVALID_ARG;
  }
  // the smallest workspace lq_lora_bwd accepts must fit; arguments the size
  // does not depend on are checked by lq_lora_bwd itself
  if (M >= 0 && r >= 1 && W0->N > 0 && W0->K > 0) {
    const size_t need = lq_workspace_size(LQ_OP_BWD_FUSED, M, W0->N, W0->K, r, 0);
    if (need > kScratchBytes) {
      lq::set_error("the backward needs %zu bytes of workspace; the static workspace holds %zu",
                    need, kScratchBytes);
      return LQ_ERR_WORKSPACE;
    }
  }
  if (lq::timing_enabled()) {  // its event pairs would be created on demand
    lq::set_error("lq_lora_bwd_noalloc needs timing off (lq_timing_enable(0))");
    return LQ_ERR_INVALID_ARG;
  }
  void* ws = nullptr;
  const int rc = scratch_ptr(&ws);
  if (rc) return rc;
  return lq_lora_bwd(dY, X, M, W0, A, B, r, scale, dt, T_saved, dX, dA, dB, accumulate, ws,
                     kScratchBytes, stream);
}
