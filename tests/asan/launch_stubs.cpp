// Stand-ins for the kernel launchers of libsanta, for a host-only build of the
// C-ABI layer (santa_api.cpp) under AddressSanitizer and UndefinedBehavior-
// Sanitizer.  No device code is built: every capacity query reports no
// resident workgroups, so a call that passes its host checks returns
// SANTA_ERR_HIP without launching anything.
#include "santa.h"
#include "launch.h"

namespace santa {
int decode_capacity(int, int, int, int, int) { return 0; }
int dense_capacity(int, int) { return 0; }
hipError_t launch_bernoulli_prep(const DecodeParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_decode(const DecodeParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_dense(const DecodeParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_pack_feature_major(const void*, void*, int, int, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_stream_read(const void*, size_t, int, uint32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gumbel(const DecodeParams&, hipStream_t) { return hipErrorNoDevice; }
}  // namespace santa

// The allocation-free entry point needs the library's device array; here it
// runs its host-side checks and stops where the array would be used.
extern "C" int santa_decode_noalloc(const santa_problem* problem, const void*, const void*, const void*,
                                    const int32_t*, int32_t S, int32_t, uint64_t, float*, int32_t*, float*,
                                    uint32_t*, void*) {
  if (!problem) return SANTA_ERR_NULL;
  const size_t need = santa::sampling_workspace_bytes(problem, S);
  if (need == 0) return SANTA_ERR_SHAPE;
  if (need > SANTA_NOALLOC_SCRATCH_BYTES) return SANTA_ERR_WORKSPACE;
  return SANTA_ERR_HIP;
}
