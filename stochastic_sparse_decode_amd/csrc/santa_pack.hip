// Relayout of a row-major K cache into 64-key feature-major tiles, the layout
// read by the Bernoulli qK^T score stage: for each (sequence, KV head) and each
// tile of 64 consecutive keys, feature i of the 64 keys is one contiguous
// 128-byte row, so a kept feature costs one row read per tile and a dropped
// feature costs nothing.  One workgroup per tile: coalesced reads of the 64
// key rows into LDS, coalesced writes of the D feature rows.
#include "device_common.h"
#include "launch.h"

namespace santa {

namespace {

template <int D>
__global__ __launch_bounds__(kThreads) void pack_kernel(const _Float16* K, _Float16* Kfm) {
  __shared__ _Float16 tile[kTile][D + 2];
  const size_t t = blockIdx.x;  // global tile index over (b, h_kv, tile)
  const _Float16* src = K + t * (size_t)(kTile * D);
  _Float16* dst = Kfm + t * (size_t)(kTile * D);
  for (int i = threadIdx.x; i < kTile * D; i += kThreads) tile[i / D][i % D] = src[i];
  __syncthreads();
  for (int i = threadIdx.x; i < kTile * D; i += kThreads) dst[i] = tile[i % kTile][i / kTile];
}

}  // namespace

hipError_t launch_pack_feature_major(const void* K, void* K_fm, int B, int Hkv, int max_n_k, int D,
                                     hipStream_t stream) {
  const size_t tiles = (size_t)B * Hkv * (max_n_k / kTile);
  if (tiles == 0) return hipSuccess;
  if (D == 64)
    hipLaunchKernelGGL(pack_kernel<64>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, (const _Float16*)K, (_Float16*)K_fm);
  else if (D == 128)
    hipLaunchKernelGGL(pack_kernel<128>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, (const _Float16*)K, (_Float16*)K_fm);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace santa
