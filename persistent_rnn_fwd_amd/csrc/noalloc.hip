// prnn_forward_dense_noalloc: the dense forward recurrence for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  It runs the same team-layout
// kernels as prnn_forward_dense, with the exchange ring in a fixed device
// array instead of a handle's buffer.
//
// The array, `scratch`, holds the ring of the largest layer the call accepts
// (32 * 2560 words: [8 XCD][2 slots][Npad], and as much again for the shared
// ring of a layer split over several XCDs per batch row) and one internal
// status word: about 320 KiB.  Each
// device the library runs on holds its own copy of it until the process ends.
// Host code never uses the array's name as an address: at a device's first
// call the address of that device's copy is looked up once (with the device
// current) and kept, and every later use goes through the kept pointer.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "host_internal.h"
#include "kernels.h"
#include "prnn.h"

namespace {

constexpr int kNoAllocMaxN = PRNN_NOALLOC_MAX_N;
constexpr size_t kRingWords = 32u * (size_t)kNoAllocMaxN;   // team ring + shared ring at N = kNoAllocMaxN
constexpr size_t kScratchWords = kRingWords + 64;            // + the internal status word (padded)
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint32_t scratch[kScratchWords];

struct DeviceState {
  bool ready = false;
  prnnStatus_t setup_status = PRNN_STATUS_SUCCESS;  // a failed set-up is returned by every call
  uint32_t* ptr = nullptr;                           // this device's copy of `scratch`
  prnn::DeviceFacts facts;
};

std::mutex g_setup_mutex;
DeviceState g_devices[kMaxDevices];

// Once per device, with it current: the device's copy of the array and the
// facts a plan needs (compute units, LDS, workgroup placement over the XCDs).
prnnStatus_t setup_device(int dev, hipStream_t stream, DeviceState** out) {
  std::lock_guard<std::mutex> lock(g_setup_mutex);
  DeviceState& d = g_devices[dev];
  *out = &d;
  if (d.ready) return d.setup_status;
  // Set-up launches a kernel and waits for it: not possible while the
  // stream is being captured (nothing is recorded; a later call retries).
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  if (cs != hipStreamCaptureStatusNone) return PRNN_STATUS_NOT_SUPPORTED;
  d.ready = true;
  hipDeviceProp_t props;
  if (hipGetDeviceProperties(&props, dev) != hipSuccess) return d.setup_status = PRNN_STATUS_INTERNAL_ERROR;
  if (std::strncmp(props.gcnArchName, "gfx950", 6) != 0 || !props.cooperativeLaunch)
    return d.setup_status = PRNN_STATUS_NOT_SUPPORTED;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return d.setup_status = PRNN_STATUS_INTERNAL_ERROR;
  }
  d.ptr = static_cast<uint32_t*>(p);
  d.facts.num_cu = props.multiProcessorCount;
  d.facts.lds_per_block = props.sharedMemPerBlock;
  // Workgroup placement over the XCDs, as prnn_create checks it (for
  // cooperative and for plain launches), with the array as the output of the
  // placement kernel (one word per workgroup).
  const int grid = d.facts.num_cu;
  auto placed = [&](bool cooperative) {
    bool ok = grid >= 8 && (size_t)grid <= kRingWords && grid <= 1024;
    uint32_t host[1024];
    if (ok) {
      uint32_t* out_words = d.ptr;
      void* args[] = {&out_words};
      const hipError_t e =
          cooperative ? hipLaunchCooperativeKernel(prnn::kPlacementKernel, dim3(grid), dim3(64), args, 0, nullptr)
                      : hipLaunchKernel(prnn::kPlacementKernel, dim3(grid), dim3(64), args, 0, nullptr);
      ok = e == hipSuccess && hipMemcpy(host, d.ptr, (size_t)grid * 4, hipMemcpyDeviceToHost) == hipSuccess;
    }
    if (ok) {
      const uint32_t c = host[0] % 8u;
      for (int i = 0; i < grid && ok; ++i) ok = host[i] < 8u && (host[i] + 8u - (uint32_t)i % 8u) % 8u == c;
    }
    (void)hipGetLastError();
    return ok;
  };
  d.facts.placement_round_robin = placed(true);
  d.facts.plain_placement = placed(false);
  const bool ok = d.facts.placement_round_robin || d.facts.plain_placement;
  return d.setup_status = ok ? PRNN_STATUS_SUCCESS : PRNN_STATUS_NOT_SUPPORTED;
}

}  // namespace

extern "C" prnnStatus_t prnn_forward_dense_noalloc(int N, int B, int T, prnnDataType_t w_type, const void* W,
                                                   const float* X, const float* h0, float* H, uint32_t* status,
                                                   hipStream_t stream) {
  if (N < 1 || B < 1 || B > 8 || T < 0) return PRNN_STATUS_BAD_PARAM;
  if (N > kNoAllocMaxN) return PRNN_STATUS_NOT_SUPPORTED;  // beyond the fixed exchange array
  if (T == 0) return PRNN_STATUS_SUCCESS;
  if (status != nullptr && (reinterpret_cast<uintptr_t>(status) & 3u) != 0) return PRNN_STATUS_BAD_PARAM;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PRNN_STATUS_INTERNAL_ERROR;
  if (dev < 0 || dev >= kMaxDevices) return PRNN_STATUS_NOT_SUPPORTED;
  DeviceState* d = nullptr;
  const prnnStatus_t st = setup_device(dev, stream, &d);
  if (st != PRNN_STATUS_SUCCESS) return st;
  uint32_t* ring = d->ptr;
  uint32_t* word = status != nullptr ? status : d->ptr + kRingWords;
  return prnn::forward_dense_on(d->facts, ring, word, N, B, T, w_type, W, X, h0, H, stream);
}
