// Paged decode without a caller workspace, for callers that cannot allocate device memory (code
// under HIP graph capture, serving loops and harnesses that forbid allocation).  The per-split
// partials that blasst_decode writes to the caller's workspace go to a file-scope device array
// instead, one copy per GPU, held until the process ends.  The kernels are the same; only the
// address of their scratch changes.
#include <mutex>

#include "common.hpp"
#include "host.hpp"

namespace {

constexpr size_t kScratchBytes = BLASST_NO_ALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The scratch array.  In host code its name is a host-side stand-in, not a device address: kernels
// and copies only ever get the address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, looked up on first use

// The current device's address of `scratch` (looked up once per device, with that device current).
blasst_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return blasst::fail(BLASST_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return blasst::fail(BLASST_ERR_UNSUPPORTED, "device %d: the scratch table covers devices 0..%d", dev,
                        kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return blasst::fail(BLASST_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                          hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return BLASST_OK;
}

}  // namespace

extern "C" blasst_status blasst_decode_no_alloc(const blasst_decode_params *p, void *stream) {
  size_t ws = 0;
  blasst_status st = blasst::decode_validate(p, &ws);
  if (st != BLASST_OK) return st;
  if (ws > kScratchBytes)
    return blasst::fail(BLASST_ERR_WORKSPACE,
                        "these params need %zu bytes of split partials; the library's scratch holds %zu "
                        "(fewer splits or sequences, or blasst_decode with a workspace)",
                        ws, kScratchBytes);
  void *ptr = nullptr;
  if (ws > 0) {
    st = scratch_address(&ptr);
    if (st != BLASST_OK) return st;
  }
  return blasst::decode_launch(p, ptr, (hipStream_t)stream);
}
