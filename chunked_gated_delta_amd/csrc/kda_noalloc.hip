// Forward entry point that allocates nothing: kda_chunk_fwd with its workspace taken from a static
// device array of this library instead of a caller buffer.
//
// For callers that cannot allocate device memory at call time (code under stream capture, tight
// serving loops, harnesses that forbid allocation).  The array is a file-scope __device__ object:
// each GPU the library runs on holds its own copy, at its own address, until the process ends.
// Host code never passes the array's name to a kernel (on the host that name is only a stand-in, not
// a device address): at a device's first call the entry point looks the address up with
// hipGetSymbolAddress, with that device current, and keeps it per device.
#include <cstdio>
#include <mutex>

#include "kda_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` on each device (null: not looked up yet)
char g_err[160] = "";

}  // namespace

extern "C" {

int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* w, const void* beta,
                          const float* S0, float g_min, int chunk, const kda_shape_t* shape, void* o,
                          float* S_final, kda_stats_t* stats, void* stream) {
  // the plan: the automatic one, except that where it would take the corrected plan (whose propagated
  // queries need 8 KiB per 32 tokens per head) the fused plan runs instead (64 KiB blocks per segment)
  if (kda_workspace_bytes(shape, chunk) == (size_t)-1) {
    // invalid shape or chunk: the full validation of the plain entry point returns the precise code
    return kda_chunk_fwd(q, k, v, w, beta, S0, g_min, chunk, shape, o, S_final, nullptr, 0, stats, stream);
  }
  kda_opts_t opts{};
  if (kda::forward_path(shape, chunk, nullptr) == kda::kModeCorr) opts.path = kda::kModeFused;
  // the scratch this call needs: host arithmetic, no HIP call
  const size_t need = kda_workspace_bytes_ex(shape, chunk, &opts);
  if (need == (size_t)-1) return KDA_ERR_ARG;
  if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return kda::record_hip_error(e);
    if (dev < 0 || dev >= kMaxDevices) {
      std::snprintf(g_err, sizeof(g_err), "device %d is beyond the %d devices the scratch table holds", dev,
                    kMaxDevices);
      return kda::record_error_text(g_err);
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return kda::record_hip_error(e);
      if (!ptr) return kda::record_error_text("hipGetSymbolAddress returned a null scratch address");
      g_scratch[dev] = ptr;
    }
    ws = g_scratch[dev];
  }
  // every segment block of the fused path is written before it is read within the call, so the
  // previous call's contents need no clearing
  return kda_chunk_fwd_ex(q, k, v, w, beta, S0, g_min, chunk, shape, o, S_final, ws, ws ? need : 0, stats, stream,
                          &opts);
}

}  // extern "C"
