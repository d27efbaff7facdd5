// Exact split-K decode attention (the in-library dense baseline).
//
// Computes softmax(scale * q K^T) V for every query head, reading all of K and
// all of V, in the split-K style of FlashDecoding: each work item (sequence,
// KV head, split of kSplit or kMinSplit keys) streams the split's K and V rows together in
// one pass, scoring its keys for the G packed query heads (the SANTA kernel's
// reduce-scatter) and keeping a running maximum, sum p and sum p * v per head
// (online softmax); the last workgroup of a KV head to finish merges the
// per-split (max, sum, vector) triples in split order:
//   out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s.
// Scheduling: persistent workgroups take items from an atomic work counter;
// there is no cross-workgroup wait in this kernel.
#include <utility>

#include "device_common.h"
#include "launch.h"
#include "score_stage.h"

namespace santa {

namespace {

template <int D, int G>
struct DenseLds {
  static constexpr size_t bytes = sizeof(float) * kWaves * G * D;  // the waves' accumulators; the merge's scales
};

struct DenseShared {
  float wmax[kWaves][8];
  float wsum[kWaves][8];
  float M[8];
  float den[8];
  int last;
  int next_item;
};



// Compile-time loop: f(std::integral_constant<int, j>) for j = 0 .. N-1.
template <typename F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Lane j of this lane's row of LPR lanes (LPR = 16: a DPP row; LPR = 8: half
// of one), by DPP row broadcasts.
template <int LPR, int J>
__device__ __forceinline__ float row_lane(float v, int lane) {
  const int x = __builtin_bit_cast(int, v);
  if constexpr (LPR == 16) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x150 + J, 0xF, 0xF, false));
  } else {
    static_assert(LPR == 8, "row width");
    const int lo = __builtin_amdgcn_update_dpp(0, x, 0x150 + J, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, x, 0x150 + 8 + J, 0xF, 0xF, false);
    return __builtin_bit_cast(float, (lane & 8) ? hi : lo);
  }
}

// Maximum over the four rows of 16 lanes at the same position, in every
// lane: a swap of the wave's halves, then of odd and even rows (VALU lane
// swaps, no LDS round trip).
__device__ __forceinline__ float max_over_rows(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the lanes of this lane's DPP row of 16 that are congruent to it
// modulo G (G a power of two, at most 8), in every lane.
template <int G>
__device__ __forceinline__ float row_sum_mod(float v) {
  if constexpr (G <= 1) v += dpp_row_ror<0x121>(v);
  if constexpr (G <= 2) v += dpp_row_ror<0x122>(v);
  if constexpr (G <= 4) v += dpp_row_ror<0x124>(v);
  return v + dpp_row_ror<0x128>(v);
}

// K and V rows of one iteration of split_pass: NB blocks of U 16-byte loads
// each, per lane.
template <int D, int G>
struct DenseBuf {
  using Gm = Geo<D, G>;
  static constexpr int NB = 2;  // blocks per register buffer
  uint4 k[NB][Gm::U], v[NB][Gm::U];
};

// Requests the K and V rows of iteration `base` of the split at k0 of KV
// head (b, hk), rows clamped to the first `lim` of the split.  The first
// iteration is requested with lim = the rows the K block holds past k0,
// before the sequence length has arrived; rows past the length get weight 0.
template <int D, int G>
__device__ __forceinline__ void dense_issue(const DecodeParams& p, int b, int hk, int k0, DenseBuf<D, G>& bf,
                                            int base, int lim) {
  using Gm = Geo<D, G>;
  constexpr int LPR = Gm::LPR, RPW = Gm::RPW, U = Gm::U, BR = Gm::BR, NB = DenseBuf<D, G>::NB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane / LPR, c = lane % LPR;
  const size_t base_row = (size_t)(b * p.Hkv + hk) * p.max_n_k + k0;
  const _Float16* Kb = (const _Float16*)p.K + base_row * D;
  const _Float16* Vb = (const _Float16*)p.V + base_row * D;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = min(base + (nb * kWaves + w) * BR + u * RPW + r, lim - 1);
      bf.k[nb][u] = load_nt((const uint4*)(Kb + (size_t)row * D + c * 8));
      bf.v[nb][u] = load_nt((const uint4*)(Vb + (size_t)row * D + c * 8));
    }
}

// The first iteration's rows taken as used (and waited for) on a path that
// scores nothing, so that the compiler requests them before it tests the item.
template <int D, int G>
__device__ __forceinline__ void dense_drop(const DenseBuf<D, G>& bf) {
#pragma unroll
  for (int nb = 0; nb < DenseBuf<D, G>::NB; ++nb)
#pragma unroll
    for (int u = 0; u < Geo<D, G>::U; ++u) asm volatile("" ::"v"(bf.k[nb][u].x), "v"(bf.v[nb][u].x));
}

// One pass over a split of `len` keys of KV head (b, hk): every wave takes
// blocks of BR consecutive rows (the waves interleave block by block),
// streams their K and V rows together with 16-byte loads (two register
// buffers of NB blocks in flight), scores the G query heads of the group (the
// SANTA score stage's reduce-scatter leaves one (row, head) score per lane),
// keeps a running maximum and sum per head (online softmax) and adds
// exp(s - m) * v into per-head accumulators.  The four waves' states are
// combined through LDS into the split's record (acc[D], m, l per head).
template <int D, int G>
__device__ __forceinline__ void split_pass(const DecodeParams& p, int b, int hk, int k0, int len, float* red,
                                           DenseShared& sh, float* rec, const DenseBuf<D, G>& first) {
  using Gm = Geo<D, G>;
  constexpr int LPR = Gm::LPR, RPW = Gm::RPW, U = Gm::U, BR = Gm::BR;
  constexpr int NB = DenseBuf<D, G>::NB;       // blocks per register buffer
  constexpr int STEP = NB * kWaves * BR;       // rows per iteration of the workgroup
  constexpr int PD = D + 2;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane / LPR, c = lane % LPR;
  const int my_u = c / G, my_g = c % G;       // this lane's score: row my_u * RPW + r of a block, head my_g
  const size_t base_row = (size_t)(b * p.Hkv + hk) * p.max_n_k + k0;
  const _Float16* Kb = (const _Float16*)p.K + base_row * D;
  const _Float16* Vb = (const _Float16*)p.V + base_row * D;
  const _Float16* qb = (const _Float16*)p.q + (size_t)(b * p.Hq + hk * G) * D;
  uint4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qv[g] = *(const uint4*)(qb + g * D + c * 8);

  float m[G], acc[G][8];
  float l = 0.f;  // sum of this lane's weights (head my_g)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
  }
  using Buf = DenseBuf<D, G>;
  // rows past the split's end re-read its last row and score -inf (weight 0),
  // so the loads are unconditional and the compiler counts them exactly
  auto issue = [&](Buf& bf, int base) { dense_issue<D, G>(p, b, hk, k0, bf, base, len); };
  auto consume = [&](const Buf& bf, int base) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float sv[LPR];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) sv[u * G + g] = dot8(bf.k[nb][u], qv[g]);
      row_reduce_scatter<LPR>(sv, lane);
      const int row = base + (nb * kWaves + w) * BR + my_u * RPW + r;
      const float sc = row < len ? sv[0] * p.scale : -INFINITY;
      // block maximum of each head (lanes congruent modulo G hold one head)
      float bm = row_max_mod<G>(sc);
      bm = max_over_rows(bm);
      float alpha[G], mine_m = 0.f, mine_a = 1.f;
      bool rescale = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float bmg = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bm), g));
        const float mn = fmaxf(m[g], bmg);
        alpha[g] = mn == -INFINITY ? 1.f : __expf(m[g] - mn);
        rescale = rescale || mn != m[g];
        m[g] = mn;
        mine_m = my_g == g ? mn : mine_m;
        mine_a = my_g == g ? alpha[g] : mine_a;
      }
      const float pw = sc == -INFINITY ? 0.f : __expf(sc - mine_m);
      l = fmaf(l, mine_a, pw);
      if (rescale) {  // wave-uniform
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] *= alpha[g];
      }
      // the V rows of the block: this lane holds features c*8.. of rows
      // u * RPW + r; the weight of (row u * RPW + r, head g) sits in lane
      // j = u * G + g of this lane's row (U * G = LPR such lanes)
      float f[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) unpack8(bf.v[nb][u], f[u]);

      static_for<LPR>([&](auto jc) {
        constexpr int J = decltype(jc)::value, u = J / G, g = J % G;
        const float wt = row_lane<LPR, J>(pw, lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(wt, f[u][e], acc[g][e]);
      });
    }
  };
  // The first iteration's rows were requested by the caller, clamped to the
  // K block.  A split shorter than one iteration then holds rows past its end
  // whose values are not ours to multiply (0 * NaN is NaN): its first rows
  // are requested again, clamped to the split.
  Buf b0 = first, b1;
  if (len < STEP) issue(b0, 0);
  for (int base = 0; base < len; base += 2 * STEP) {
    issue(b1, base + STEP);
    consume(b0, base);
    issue(b0, base + 2 * STEP);
    consume(b1, base + STEP);
  }

  // combine: the RPW key-row groups of a wave (lanes with the same c), the
  // lanes of each head for l, then the four waves through LDS.  The row
  // groups are summed in registers (reduce-scatter): a swap of the wave's
  // halves pairs feature e with e + 4 (the lower half keeps the sums of 0..3,
  // the upper those of 4..7), a swap of odd and even rows of 16 pairs the
  // remaining j with j + 2, and for D = 64 (rows of 8 lanes) a rotation adds
  // the two halves of each row of 16.  Lane (r, c) then holds the wave's
  // totals of features c*8 + 2r, c*8 + 2r + 1 (D = 128) or c*8 + r (D = 64).
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float h4[4], h2[2];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[g][e]), __float_as_uint(acc[g][e + 4]), false, false);
      h4[e] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(h4[e]), __float_as_uint(h4[e + 2]), false, false);
      h2[e] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    }
    float* dst = red + (w * G + g) * D + c * 8;
    if constexpr (D == 128) {
      *(float2*)(dst + 2 * r) = make_float2(h2[0], h2[1]);
    } else {
      static_assert(D == 64, "head dimension");
      const float s0 = h2[0] + dpp_row_ror<0x128>(h2[0]);
      const float s1 = h2[1] + dpp_row_ror<0x128>(h2[1]);
      dst[r] = (r & 1) ? s1 : s0;
    }
  }
  float lw = row_sum_mod<G>(l);
  {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(lw), __float_as_uint(lw), false, false);
    lw = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(lw), __float_as_uint(lw), false, false);
    lw = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  }
  if (lane < G) {
    sh.wmax[w][lane] = m[0];
#pragma unroll
    for (int g = 1; g < G; ++g)
      if (lane == g) sh.wmax[w][lane] = m[g];
    sh.wsum[w][lane] = lw;  // lane g holds head g (lanes congruent to g modulo G)
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += kThreads) {
    const int g = i / D, d = i % D;
    float M = sh.wmax[0][g];
#pragma unroll
    for (int x = 1; x < kWaves; ++x) M = fmaxf(M, sh.wmax[x][g]);
    float v = 0.f;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) {
      const float mx = sh.wmax[x][g];
      v += mx == -INFINITY ? 0.f : red[(x * G + g) * D + d] * __expf(mx - M);
    }
    store_dev(rec + g * PD + d, v);
  }
  if (tid < G) {
    float M = sh.wmax[0][tid];
#pragma unroll
    for (int x = 1; x < kWaves; ++x) M = fmaxf(M, sh.wmax[x][tid]);
    float lt = 0.f;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) {
      const float mx = sh.wmax[x][tid];
      lt += mx == -INFINITY ? 0.f : sh.wsum[x][tid] * __expf(mx - M);
    }
    store_dev(rec + tid * PD + D, M);
    store_dev(rec + tid * PD + D + 1, lt);
  }
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void dense_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = (float*)smem;  // [kWaves][G][D] the waves' accumulators, then the merge's per-split scales
  __shared__ DenseShared sh;
  constexpr int LPR = D / 8, RPW = 64 / LPR, UV = 8;
  constexpr int PD = D + 2;  // partial record: acc[D], m, l
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane / LPR, c = lane % LPR;
  int item = blockIdx.x;

  while (item < p.total_items) {
    const int group = item / p.ns, s = item % p.ns;
    const int b = group / p.Hkv, hk = group % p.Hkv, h0 = hk * G;
    // the length is a scalar read (it does not change during the kernel), and
    // the split's first K and V rows are requested before it is used: they
    // need only the item's place and the K block's row count
    const int n = *(const __attribute__((address_space(4))) int32_t*)(p.n_k + b);
    const int k0 = s * p.split;
    DenseBuf<D, G> first;
    dense_issue<D, G>(p, b, hk, k0, first, 0, min(p.split, p.max_n_k - k0));
    const bool valid = n >= 1 && n <= p.max_n_k;
    const int nsg = valid ? (n + p.split - 1) / p.split : 0;

    if (!valid) {
      dense_drop<D, G>(first);
      if (s == 0)
        for (int i = tid; i < G * D; i += kThreads) p.out[(size_t)(b * p.Hq + h0) * D + i] = __builtin_nanf("");
    } else if (s >= nsg) {
      dense_drop<D, G>(first);
    } else {
      const int len = min(p.split, n - k0);
      split_pass<D, G>(p, b, hk, k0, len, red, sh, p.ws.partial + (size_t)(group * p.ns + s) * G * PD, first);
      wait_memory();
      __syncthreads();
      // arrival counter of the group (zero at rest: the last arrival resets it)
      if (tid == 0) sh.last = atomic_add_dev(p.ws.arrive + group, 1u) == (uint32_t)(nsg - 1);
      __syncthreads();
      if (sh.last) {
        // out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s, split order
        const float* gp = p.ws.partial + (size_t)group * p.ns * G * PD;
        constexpr int CH = 32;                // splits merged per pass
        constexpr int OPT = (G * D + kThreads - 1) / kThreads;
        float t[OPT][CH];  // one pass's partial vectors, all loads in flight at once
        auto load_pass = [&](int x0) {
#pragma unroll
          for (int o = 0; o < OPT; ++o) {
            const int i = min(tid + o * kThreads, G * D - 1);
            const int g = i / D, d = i % D;
#pragma unroll
            for (int u = 0; u < CH; ++u) t[o][u] = load_dev(gp + (size_t)min(x0 + u, nsg - 1) * G * PD + g * PD + d);
          }
        };
        // the first pass's vectors and its splits' (m, l) are requested
        // together, with the maxima of the later splits, so that all of them
        // arrive in one round trip: thread tid < CH * G holds (m, l) of split
        // x0 + tid / G, head tid % G of the pass
        load_pass(0);
        auto load_ml = [&](int x0, float& mx, float& lx) {
          const int x = x0 + tid / G, g = tid % G;
          mx = -INFINITY;
          lx = 0.f;
          if (tid < CH * G && x < nsg) {
            const float* rec = gp + (size_t)x * G * PD + g * PD;
            mx = load_dev(rec + D);
            lx = load_dev(rec + D + 1);
          }
        };
        float mx, lx;
        load_ml(0, mx, lx);
        // the maximum over every split: this pass's from mx, later ones read here
        float mo = mx;
        for (int x = CH + tid / G; x < nsg; x += kThreads / G) mo = fmaxf(mo, load_dev(gp + (size_t)x * G * PD + (tid % G) * PD + D));
        // lanes congruent modulo G hold one head: rows of 16, then across rows
        mo = max_over_rows(row_max_mod<G>(mo));
        if (lane < G) sh.wmax[w][lane] = mo;
        if (tid < G) sh.den[tid] = 0.f;
        __syncthreads();
        if (tid < G) {
          float m = sh.wmax[0][tid];
#pragma unroll
          for (int x = 1; x < kWaves; ++x) m = fmaxf(m, sh.wmax[x][tid]);
          sh.M[tid] = m;
        }
        __syncthreads();
        float* scl = red;                     // [CH][G] e^(m_s - M)
        float* lsc = red + CH * G;            // [CH][G] l_s e^(m_s - M)
        static_assert(2 * CH * G <= kWaves * G * D, "the merge's scales fit the accumulator area");
        float num[OPT];
#pragma unroll
        for (int o = 0; o < OPT; ++o) num[o] = 0.f;
        for (int x0 = 0; x0 < nsg; x0 += CH) {
          if (x0 > 0) {
            load_pass(x0);
            load_ml(x0, mx, lx);
          }
          if (tid < CH * G) {
            const float sc = mx == -INFINITY ? 0.f : expf(mx - sh.M[tid % G]);
            scl[tid] = sc;
            lsc[tid] = lx * sc;
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
