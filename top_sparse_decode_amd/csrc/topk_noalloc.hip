// topk_select_noalloc: the exact top-k of topk_select for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid allocation). The selection's workspace lives in one
// file-scope device array of fixed size instead of a caller buffer; the
// kernels are topk_select's own and take that array's device address the
// way they take a caller workspace.
//
// The array's name is a host-side stand-in, not a device address: host code
// uses only the address hipGetSymbolAddress returns, fetched once per device
// (with that device current) on the first call there and kept per device.
// Every call on a device shares its array; the histograms the selection
// needs zeroed are cleared by a kernel at the start of every call (no
// memset node), and calls that overlap on one device race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "tsd.h"

namespace {

constexpr size_t kScratchBytes = size_t{8} << 20;  // 8 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array, or nullptr (with *err set)
// when the runtime cannot give it.
void* scratch_address(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t topk_select_noalloc_max_bytes(void) { return kScratchBytes; }

int topk_select_noalloc(const float* scores, int64_t stride, int rows,
                        const int32_t* row_lens, int max_len, int k,
                        int32_t* idx, int32_t* count, hipStream_t stream) {
  if (rows < 0 || max_len < 0 || stride < 1 || stride < max_len)
    return TSD_E_SHAPE;
  if (k < 1 || k > TSD_MAX_TOPK) return TSD_E_K;
  if (rows > 65535 || max_len > tsd::topk_max_len()) return TSD_E_UNSUPPORTED;
  if (rows == 0) return TSD_OK;
  if (!scores || !row_lens || !idx) return TSD_E_NULL;
  if (tsd::topk_workspace(rows, max_len, k) > kScratchBytes)
    return TSD_E_SCRATCH;
  hipError_t e = hipSuccess;
  void* ws = scratch_address(&e);
  if (!ws) return static_cast<int>(e);
  e = tsd::launch_topk(scores, stride, rows, row_lens, max_len, k, idx, count,
                       ws, /*zeroed=*/false, stream);
  return e == hipSuccess ? TSD_OK : static_cast<int>(e);
}

}  // extern "C"
