// Exact split-K decode attention (the in-library dense baseline).
//
// Computes softmax(scale * q K^T) V for every query head, reading all of K and
// all of V, in the split-K style of FlashDecoding: each work item (sequence,
// KV head, split of kSplit keys) scores its keys for the G packed query heads
// (same score stage as the SANTA kernel), keeps the scores in LDS, forms
// p = exp(s - local max) and streams the split's V rows once, accumulating
// sum p * v and sum p.  The last workgroup of a KV head to finish merges the
// per-split (max, sum, vector) triples in split order:
//   out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s.
// Scheduling: persistent workgroups take items from an atomic work counter;
// there is no cross-workgroup wait in this kernel.
#include "device_common.h"
#include "launch.h"
#include "score_stage.h"

namespace santa {

namespace {

constexpr int kPad = pad_of<kSplit>();

template <int D, int G>
struct DenseLds {
  static constexpr size_t p_bytes = sizeof(float) * G * kPad;
  static constexpr size_t red_bytes = sizeof(float) * kWaves * G * D;
  static constexpr size_t bytes = p_bytes + red_bytes;
};

struct DenseShared {
  float wmax[kWaves][8];
  float wsum[kWaves][8];
  float M[8];
  float den[8];
  int last;
  int next_item;
};



template <int D, int G>
__global__ __launch_bounds__(kThreads) void dense_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* P = (float*)smem;                                  // [G][kPad] scores, then weights
  float* red = (float*)(smem + DenseLds<D, G>::p_bytes);    // [kWaves][G*D]
  __shared__ DenseShared sh;
  constexpr int LPR = D / 8, RPW = 64 / LPR, UV = 8;
  constexpr int PD = D + 2;  // partial record: acc[D], m, l
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane / LPR, c = lane % LPR;
  int item = blockIdx.x;

  while (item < p.total_items) {
    const int group = item / p.ns, s = item % p.ns;
    const int b = group / p.Hkv, hk = group % p.Hkv, h0 = hk * G;
    const int n = p.n_k[b];
    const bool valid = n >= 1 && n <= p.max_n_k;
    const int nsg = valid ? (n + kSplit - 1) / kSplit : 0;

    if (!valid) {
      if (s == 0)
        for (int i = tid; i < G * D; i += kThreads) p.out[(size_t)(b * p.Hq + h0) * D + i] = __builtin_nanf("");
    } else if (s < nsg) {
      const int k0 = s * kSplit;
      const int len = min(kSplit, n - k0);
      float mx[G];
      score_rowmajor<D, G>(p, b, hk, k0, len, P, mx);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m = wave_max_masked(mx[g], 1);
        if (lane == 0) sh.wmax[w][g] = m;
      }
      __syncthreads();
      // weights p_j = exp(s_j - m) in place, and their sum per head
      float m_h[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        m_h[g] = sh.wmax[0][g];
#pragma unroll
        for (int x = 1; x < kWaves; ++x) m_h[g] = fmaxf(m_h[g], sh.wmax[x][g]);
      }
      float lsum[G];
#pragma unroll
      for (int g = 0; g < G; ++g) lsum[g] = 0.f;
      for (int j = tid; j < len; j += kThreads) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float e = expf(P[g * kPad + lidx(j)] - m_h[g]);
          P[g * kPad + lidx(j)] = e;
          lsum[g] += e;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float v = lsum[g];
        for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
        if (lane == 0) sh.wsum[w][g] = v;
      }
      __syncthreads();

      // stream the split's V rows once: acc_g += p_gj * v_j
      const _Float16* Vb = (const _Float16*)p.V + ((size_t)(b * p.Hkv + hk) * p.max_n_k + k0) * D;
      float acc[G][8];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
      constexpr int ROWS_IT = UV * kWaves * RPW;
      // two register buffers in a ping-pong loop: the rows of the next
      // iteration are in flight while this iteration's FMAs run.  Loads are
      // unconditional (rows past the end re-read the last row, weight 0), so
      // the compiler counts outstanding loads exactly.
      static_assert(kSplit % (2 * ROWS_IT) == 0, "iterations come in pairs");
      uint4 va[UV], vb[UV];
      auto issue = [&](uint4 (&bb)[UV], int base) {
#pragma unroll
        for (int x = 0; x < UV; ++x) {
          const int row = min(base + (x * kWaves + w) * RPW + r, len - 1);
          bb[x] = load_nt((const uint4*)(Vb + (size_t)row * D + c * 8));
        }
      };
      auto consume = [&](const uint4 (&bb)[UV], int base) {
#pragma unroll
        for (int x = 0; x < UV; ++x) {
          const int row = base + (x * kWaves + w) * RPW + r;
          float f[8];
          unpack8(bb[x], f);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float pw = row < len ? P[g * kPad + lidx(row)] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pw, f[e], acc[g][e]);
          }
        }
      };
      issue(va, 0);
      for (int base = 0; base < len; base += 2 * ROWS_IT) {
        issue(vb, base + ROWS_IT);
        consume(va, base);
        issue(va, base + 2 * ROWS_IT);
        consume(vb, base + ROWS_IT);
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          for (int m = LPR; m < 64; m <<= 1) acc[g][e] += __shfl_xor(acc[g][e], m, 64);
      if (r == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) red[w * G * D + g * D + c * 8 + e] = acc[g][e];
      }
      __syncthreads();
      float* part = p.ws.partial + (size_t)(group * p.ns + s) * G * PD;
      for (int i = tid; i < G * D; i += kThreads) {
        float v = red[i];
#pragma unroll
        for (int x = 1; x < kWaves; ++x) v += red[x * G * D + i];
        store_dev(part + (i / D) * PD + (i % D), v);
      }
      if (tid < G) {
        float l = sh.wsum[0][tid];
#pragma unroll
        for (int x = 1; x < kWaves; ++x) l += sh.wsum[x][tid];
        float mh = sh.wmax[0][tid];
#pragma unroll
        for (int x = 1; x < kWaves; ++x) mh = fmaxf(mh, sh.wmax[x][tid]);
        store_dev(part + tid * PD + D, mh);
        store_dev(part + tid * PD + D + 1, l);
      }
      wait_memory();
      __syncthreads();
      // arrival counter of the group (zero at rest: the last arrival resets it)
      if (tid == 0) sh.last = atomic_add_dev(p.ws.arrive + group, 1u) == (uint32_t)(nsg - 1);
      __syncthreads();
      if (sh.last) {
        // out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s, split order
        const float* gp = p.ws.partial + (size_t)group * p.ns * G * PD;
        float mg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) mg[g] = -INFINITY;
        for (int x = tid; x < nsg; x += kThreads)
#pragma unroll
          for (int g = 0; g < G; ++g) mg[g] = fmaxf(mg[g], load_dev(gp + (size_t)x * G * PD + g * PD + D));
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float m = wave_max_masked(mg[g], 1);
          if (lane == 0) sh.wmax[w][g] = m;
        }
        if (tid < G) sh.den[tid] = 0.f;
        __syncthreads();
        if (tid < G) {
          float m = sh.wmax[0][tid];
#pragma unroll
          for (int x = 1; x < kWaves; ++x) m = fmaxf(m, sh.wmax[x][tid]);
          sh.M[tid] = m;
        }
        __syncthreads();
        constexpr int CH = 32;                // splits merged per pass
        float* scl = P;                       // [CH][G] e^(m_s - M)
        float* lsc = P + CH * G;              // [CH][G] l_s e^(m_s - M)
        constexpr int OPT = (G * D + kThreads - 1) / kThreads;
        float num[OPT];
#pragma unroll
        for (int o = 0; o < OPT; ++o) num[o] = 0.f;
        for (int x0 = 0; x0 < nsg; x0 += CH) {
          float t[OPT][CH];  // this pass's partial vectors, all loads in flight at once
#pragma unroll
          for (int o = 0; o < OPT; ++o) {
            const int i = min(tid + o * kThreads, G * D - 1);
            const int g = i / D, d = i % D;
#pragma unroll
            for (int u = 0; u < CH; ++u) t[o][u] = load_dev(gp + (size_t)min(x0 + u, nsg - 1) * G * PD + g * PD + d);
          }
          if (tid < CH * G) {
            const int x = x0 + tid / G, g = tid % G;
            float sc = 0.f, l = 0.f;
            if (x < nsg) {
              const float* rec = gp + (size_t)x * G * PD + g * PD;
              sc = expf(load_dev(rec + D) - sh.M[g]);
              l = load_dev(rec + D + 1);
            }
            scl[tid] = sc;
            lsc[tid] = l * sc;
          }
          __syncthreads();
#pragma unroll
          for (int o = 0; o < OPT; ++o) {
            const int g = min(tid + o * kThreads, G * D - 1) / D;
#pragma unroll
            for (int u = 0; u < CH; ++u) num[o] = fmaf(t[o][u], scl[u * G + g], num[o]);  // scl = 0 past nsg
          }
          if (tid < G) {
            float dsum = sh.den[tid];
            for (int u = 0; u < CH; ++u) dsum += lsc[u * G + tid];
            sh.den[tid] = dsum;
          }
          __syncthreads();
        }
#pragma unroll
        for (int o = 0; o < OPT; ++o) {
          const int i = tid + o * kThreads;
          if (i < G * D) p.out[(size_t)(b * p.Hq + h0) * D + i] = num[o] / sh.den[i / D];
        }
        if (tid == 0) store_dev(p.ws.arrive + group, 0u);
      }
    }

    if (p.grid >= p.total_items) break;
    __syncthreads();
    if (tid == 0) {
      const uint32_t t = atomic_add_dev(p.ws.work_ctr, 1u);
      sh.next_item = p.grid + (int)t;
      if (t == (uint32_t)(p.total_items - 1)) store_dev(p.ws.work_ctr, 0u);
    }
    __syncthreads();
    item = sh.next_item;
  }
}

template <int D, int G>
int capacity_t() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  auto fn = dense_kernel<D, G>;
  const size_t lds = DenseLds<D, G>::bytes;
  (void)hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess) return 0;
  return per_cu * cus;
}

template <int D, int G>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const size_t lds = DenseLds<D, G>::bytes;
  hipLaunchKernelGGL((dense_kernel<D, G>), dim3(p.grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

int dense_capacity(int D, int G) {
#define SANTA_CASE(DD, GG) \
  if (D == DD && G == GG) return capacity_t<DD, GG>();
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return 0;
}

hipError_t launch_dense(const DecodeParams& p, hipStream_t stream) {
#define SANTA_CASE(DD, GG) \
  if (p.D == DD && p.G == GG) return launch_t<DD, GG>(p, stream);
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return hipErrorInvalidValue;
}

}  // namespace santa
