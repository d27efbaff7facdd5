// SANTA with i.i.d. draws by the Gumbel-max trick (sampling mode 3): the
// alternative to the inverse-CDF sampler named beside the Bernoulli budget
// variant.  Draw k selects argmax_j (s_j + g_kj), g_kj = -log(-log u_kj), which
// falls on key j with probability softmax(s)_j; the S draws are i.i.d. from the
// post-softmax distribution, like mode 0, with other random numbers.
//
// u_kj: output word (j & 3) of Philox4x32-10 at counter (j >> 2, row, 'GUMB',
// k), key (seed lo, seed hi), row = b * H_q + h, mapped into the open interval
// as ((x >> 9) + 1/2) * 2^-23, which fp32 holds exactly, in [2^-24, 1 - 2^-24],
// so both logarithms are finite.  Every (draw, key) pair needs its own variate, so
// the sampler does S * n_k generator and logarithm evaluations per query head
// (arithmetic-bound; the inverse CDF needs S uniforms).
//
// Three launches:
//   gumbel_clear   the per-(head, draw) winners are set to 0;
//   gumbel_kernel  work item = (sequence, KV head, split of kSplit keys): the
//                  split's keys are scored for the G heads of the group (the
//                  decode kernels' score stage), then each (head, draw) pair
//                  takes the maximum of s_j + g_kj over the split's keys and
//                  merges it into the pair's winner with a 64-bit atomic max
//                  of (order-preserving bits of the value, ~key): a larger
//                  value wins, and the smaller key on a tie;
//   gumbel_gather  one workgroup per query head: the S winning keys, sorted,
//                  their value rows summed exactly (fp64: fp16 products and
//                  sums of at most SANTA_MAX_S rows are exact) and rounded once
//                  after the division by S.
#include "device_common.h"
#include "launch.h"
#include "score_stage.h"

namespace santa {

namespace {

constexpr uint32_t kTagGumbel = 0x47554D42u;  // 'GUMB'

// 32-bit key whose unsigned order is the order of the fp32 values.
__device__ __forceinline__ uint32_t order_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kThreads) void gumbel_clear(uint64_t* win, size_t n) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads) win[i] = 0ull;
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void gumbel_kernel(DecodeParams p, uint64_t* win) {
  constexpr int kPad = pad_of<kSplit>();
  __shared__ __align__(16) float sc[G * kPad];
  const int tid = threadIdx.x;
  const int S = p.S;
  const uint32_t k0s = (uint32_t)(p.seed & 0xffffffffu), k1s = (uint32_t)(p.seed >> 32);
  for (int item = blockIdx.x; item < p.total_items; item += gridDim.x) {
    const int group = item / p.ns, s = item % p.ns;
    const int b = group / p.Hkv, hk = group % p.Hkv;
    const int n = p.n_k[b];
    if (n < 1 || n > p.max_n_k || s * kSplit >= n) continue;  // invalid lengths: the gather writes NaN
    const int k0 = s * kSplit, len = min(kSplit, n - k0);
    float mx[G];
    score_rowmajor<D, G, 16>(p, b, hk, k0, len, sc, mx);
    (void)mx;
    __syncthreads();
    if (p.scores_out) write_scores<G>(p, b, hk, k0, len, sc);
    // (head, draw) pairs over the workgroup's lanes; with fewer pairs than
    // lanes each pair's keys are cut into `parts` ranges (multiples of 8
    // keys), each lane merging its own range's maximum (the atomic maximum is
    // associative).  The lanes of a wave read a few score slots at a time,
    // which LDS broadcasts; two generator blocks per step keep two
    // independent Philox chains in flight.
    const int pairs = G * S;
    int parts = 1;
    while (pairs * parts * 2 <= kThreads && parts < kSplit / 8) parts *= 2;
    const int chunk = ((len + parts - 1) / parts + 7) & ~7;
    for (int t = tid; t < pairs * parts; t += kThreads) {
      const int pr = t % pairs, part = t / pairs;
      const int g = pr % G, k = pr / G;
      const uint32_t row = (uint32_t)(b * p.Hq + hk * G + g);
      const float* cg = sc + g * kPad;
      const int jb = part * chunk, je = min(len, jb + chunk);
      float best = -INFINITY;
      int bi = -1;
      for (int j = jb; j < je; j += 8) {
        const uint4 x0 = philox4x32_10(make_uint4((uint32_t)(k0 + j) >> 2, row, kTagGumbel, (uint32_t)k), k0s, k1s);
        const uint4 x1 = philox4x32_10(make_uint4((uint32_t)(k0 + j + 4) >> 2, row, kTagGumbel, (uint32_t)k), k0s, k1s);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int jj = j + e;
          const uint32_t w = word_of(e < 4 ? x0 : x1, e & 3);
          const float u = ((float)(w >> 9) + 0.5f) * 0x1.0p-23f;  // exact in fp32
          const float v = cg[lidx(min(jj, len - 1))] - __logf(-__logf(u));
          const bool better = jj < je && v > best;  // strict: the first (smaller) key keeps a tie
          best = better ? v : best;
          bi = better ? jj : bi;
        }
      }
      if (bi >= 0) {
        const uint64_t packed = ((uint64_t)order_bits(best) << 32) | (uint64_t)(~(uint32_t)(k0 + bi));
        __hip_atomic_fetch_max(win + (size_t)row * S + k, packed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // the score buffer is reused by the next item
  }
}

// One workgroup per query head: the winners' keys, sorted ascending (LDS
// bitonic sort over the next power of two of S), the gathered rows summed in
// fp64 (exact) and rounded once.
template <int D>
__global__ __launch_bounds__(kThreads) void gumbel_gather(DecodeParams p, const uint64_t* win) {
  __shared__ int keys[kMaxS];
  __shared__ double part[kThreads / D > 0 ? kThreads / D : 1][D];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;  // b * H_q + h
  const int b = row / p.Hq, h = row % p.Hq, hk = h / p.G;
  const int S = p.S;
  const int n = p.n_k[b];
  if (n < 1 || n > p.max_n_k) {
    for (int i = tid; i < D; i += kThreads) p.out[(size_t)row * D + i] = __builtin_nanf("");
    if (p.idx_out)
      for (int i = tid; i < S; i += kThreads) p.idx_out[(size_t)row * S + i] = -1;
    return;
  }
  int P2 = 1;
  while (P2 < S) P2 <<= 1;
  for (int i = tid; i < P2; i += kThreads)
    keys[i] = i < S ? (int)~(uint32_t)(win[(size_t)row * S + i] & 0xffffffffull) : 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= P2; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P2; i += kThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const int a = keys[i], c = keys[j];
          if ((a > c) == up) {
            keys[i] = c;
            keys[j] = a;
          }
        }
      }
      __syncthreads();
    }
  if (p.idx_out)
    for (int i = tid; i < S; i += kThreads) p.idx_out[(size_t)row * S + i] = keys[i];
  // exact sum: thread (r, d) adds rows r, r + R, ... of feature d in order
  constexpr int R = kThreads / D > 0 ? kThreads / D : 1;
  const int r = tid / D, d = tid % D;
  const _Float16* Vb = (const _Float16*)p.V + (size_t)(b * p.Hkv + hk) * p.max_n_k * D;
  double acc = 0.0;
  if (r < R)
    for (int i = r; i < S; i += R) acc += (double)(float)Vb[(size_t)keys[i] * D + d];
  if (r < R) part[r][d] = acc;
  __syncthreads();
  if (tid < D) {
    double t = 0.0;
#pragma unroll
    for (int x = 0; x < R; ++x) t += part[x][tid];
    p.out[(size_t)row * D + tid] = (float)(t / (double)S);
  }
}

template <int D, int G>
hipError_t launch_gumbel_t(const DecodeParams& p, hipStream_t stream) {
  uint64_t* win = p.ws.acc;  // [B][H_q][S] winners
  const size_t n = (size_t)p.B * p.Hq * p.S;
  hipLaunchKernelGGL(gumbel_clear, dim3((unsigned)((n + kThreads - 1) / kThreads < 1024 ? (n + kThreads - 1) / kThreads
                                                                                           : 1024)),
                     dim3(kThreads), 0, stream, win, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gumbel_kernel<D, G>), dim3(p.grid), dim3(kThreads), 0, stream, p, win);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gumbel_gather<D>), dim3(p.B * p.Hq), dim3(kThreads), 0, stream, p, (const uint64_t*)win);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gumbel(const DecodeParams& p, hipStream_t stream) {
#define SANTA_CASE(DD, GG) \
  if (p.D == DD && p.G == GG) return launch_gumbel_t<DD, GG>(p, stream);
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return hipErrorInvalidValue;
}

}  // namespace santa
