// santa_decode_noalloc: santa_decode with its workspace in device memory that
// the library owns, for callers that cannot allocate (code under HIP graph
// capture, serving loops, harnesses that forbid allocation).
//
// The workspace is the file-scope array `scratch` below: each GPU the library
// runs on holds its own copy (kScratchBytes, until the process ends).  In host
// code the array's name is only a stand-in for the device symbol, so its device
// address on the current GPU is taken once per device with
// hipGetSymbolAddress and that pointer is what the kernels receive.  Every
// call on a GPU shares that GPU's array: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "santa.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = SANTA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each GPU, once taken

// Clears the error word of the workspace header.  The array starts zero-filled
// (static storage); this makes the first call's error word zero whatever an
// earlier process state was, and does not touch the launch counter (a replay of
// a captured first call must not repeat launch tags).
__global__ void clear_error_word(unsigned int* err) {
  if (threadIdx.x == 0) err[0] = 0u;
}

// Device address of the current GPU's array (nullptr on a HIP error); the
// first call on a device also enqueues the clear of its error word.
void* scratch_on_current_device(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    hipLaunchKernelGGL(clear_error_word, dim3(1), dim3(64), 0, stream, (unsigned int*)ptr);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int santa_decode_noalloc(const santa_problem* problem, const void* q, const void* K, const void* V,
                                    const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, float* out,
                                    int32_t* indices_out, float* scores_out, uint32_t* error_flags, void* stream) {
  if (!problem) return SANTA_ERR_NULL;
  const size_t need = santa::sampling_workspace_bytes(problem, S);
  if (need == 0) return SANTA_ERR_SHAPE;
  if (need > kScratchBytes) return SANTA_ERR_WORKSPACE;  // beyond the library's array
  void* ws = scratch_on_current_device((hipStream_t)stream);
  if (!ws) return SANTA_ERR_HIP;
  return santa::decode_on(problem, q, K, V, n_k, S, mode, seed, out, indices_out, scores_out, ws, kScratchBytes,
                          error_flags, stream);
}
