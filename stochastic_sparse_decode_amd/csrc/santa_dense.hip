// Exact split-K decode attention (the in-library dense baseline).
//
// Computes softmax(scale * q K^T) V for every query head, reading all of K and
// all of V, in the split-K style of FlashDecoding: each work item (sequence,
// KV head, split of kSplit or kMinSplit keys) streams the split's K and V rows together in
// one pass, scoring its keys for the G packed query heads (the SANTA kernel's
// reduce-scatter) and keeping a running maximum, sum p and sum p * v per head
// (online softmax).  The per-split (max, sum, vector) triples merge in split
// order:
//   out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s.
// Two schedules:
//  - every item resident at once (one workgroup each): the splits of a KV
//    head store their triples as tagged words and each split merges a 1/ns
//    share of the head group's features from all of them (a bounded wait on
//    the other splits' records, which are all being computed);
//  - else persistent workgroups take items from an atomic work counter, and
//    the last split of a KV head to finish merges every triple (no
//    cross-workgroup wait).
#include <algorithm>
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
  uint32_t epoch;  // launch tag (exchange merge)
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
// each, per lane.  A block of G = 1 at d = 128 is already 64 rows (16 loads
// of K and 16 of V per lane), so its buffer holds one.
template <int D, int G>
struct DenseBuf {
  using Gm = Geo<D, G>;
  static constexpr int NB = Gm::U >= 16 ? 1 : 2;  // blocks per register buffer
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
// exp(s - m) * v into per-head accumulators.  Each wave leaves its state in
// LDS (accumulators in red, maximum and sum per head in sh); finish_split
// combines the four.
template <int D, int G>
__device__ __forceinline__ void split_pass(const DecodeParams& p, int b, int hk, int k0, int len, float* red,
                                           DenseShared& sh, const DenseBuf<D, G>& first, bool first_to_block) {
  using Gm = Geo<D, G>;
  constexpr int LPR = Gm::LPR, RPW = Gm::RPW, U = Gm::U, BR = Gm::BR;
  constexpr int NB = DenseBuf<D, G>::NB;       // blocks per register buffer
  constexpr int STEP = NB * kWaves * BR;       // rows per iteration of the workgroup
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
      if constexpr (G == 1) {
        // one head: each row's values are unpacked where they are used (the
        // 16 rows of a lane unpacked at once would take 128 registers)
        static_for<LPR>([&](auto jc) {
          constexpr int J = decltype(jc)::value;
          const float wt = row_lane<LPR, J>(pw, lane);
          float fj[8];
          unpack8(bf.v[nb][J], fj);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[0][e] = fmaf(wt, fj[e], acc[0][e]);
        });
      } else {
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
    }
  };
  // The first iteration's rows were requested by the caller, clamped to the
  // split, or (first_to_block) to the K block.  A split shorter than one
  // iteration then holds rows past its end whose values are not ours to
  // multiply (0 * NaN is NaN): its first rows are requested again, clamped to
  // the split.
  Buf b0 = first, b1;
  if (first_to_block && len < STEP) issue(b0, 0);
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
}

// Where a split's combined state goes.
enum Finish { kFloatRecord = 0, kTaggedRecord = 1, kOutput = 2 };

// After split_pass and a barrier: the four waves' states combine into the
// split's maximum M, sum l and vector acc per head, written as a float record
// (acc[D], M, l per head), as the same record in tagged words (tag:32 | value
// bits), or, when the split is its group's only one, as the output acc / l.
template <int D, int G>
__device__ __forceinline__ void finish_split(const float* red, DenseShared& sh, int how, float* rec, uint64_t* xr,
                                             uint32_t tag, float* outp) {
  constexpr int PD = D + 2;
  const int tid = threadIdx.x;
  const uint64_t t = (uint64_t)tag << 32;
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
    if (how == kFloatRecord) {
      store_dev(rec + tid * PD + D, M);
      store_dev(rec + tid * PD + D + 1, lt);
    } else if (how == kTaggedRecord) {
      store_dev(xr + tid * PD + D, t | __float_as_uint(M));
      store_dev(xr + tid * PD + D + 1, t | __float_as_uint(lt));
    } else {
      sh.den[tid] = lt;
    }
  }
  if (how == kOutput) __syncthreads();
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
    if (how == kFloatRecord) store_dev(rec + g * PD + d, v);
    else if (how == kTaggedRecord) store_dev(xr + g * PD + d, t | __float_as_uint(v));
    else outp[i] = v / sh.den[g];
  }
}

// Sum over the 64 lanes of a wave, returned in every lane, in a fixed order:
// DPP row shifts (an empty source adds 0) and row broadcasts leave the sum in
// lane 63, which is then read as a scalar.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add_step(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                   0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add_step<0x111, 0xF>(v);  // row_shr:1
  v = dpp_add_step<0x112, 0xF>(v);  // row_shr:2
  v = dpp_add_step<0x114, 0xF>(v);  // row_shr:4
  v = dpp_add_step<0x118, 0xF>(v);  // row_shr:8
  v = dpp_add_step<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_add_step<0x143, 0xC>(v);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Merge by exchange, for split s of a group of nsg > 1 splits whose
// workgroups are all resident: split s produces features [f0, f1) of the
// group's F = G * D outputs (head f / D, feature f mod D) from every split's
// tagged record,
//   out_f = sum_x e^(m_x - M) acc_x,f / sum_x e^(m_x - M) l_x  (x in split order).
// Every split stores its record before it reads, so every wait ends; a wait
// is bounded regardless (kSpinLimit rounds, then an error bit).  A word is
// accepted only with this launch's tag; a thread re-reads only the words it
// has not yet seen.
template <int D, int G>
__device__ __forceinline__ void exchange_merge(const DecodeParams& p, const uint64_t* grec, int s, int nsg,
                                               uint32_t tag, float* vals, float2* xml, float* scl, float* den,
                                               float* outp) {
  constexpr int F = G * D, PD = D + 2, RW = G * PD;  // 8-byte words per split record
  constexpr int NV = (F + kMaxExchSplits + kThreads - 1) / kThreads;  // value words per thread
  static_assert(2 * kMaxExchSplits <= kThreads, "one (m, l) pair per thread");
  static_assert(kMaxExchSplits <= 3 * 64, "the values fit the accumulator area");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int f0 = s * F / nsg, f1 = (s + 1) * F / nsg, chunk = f1 - f0;
  if (chunk == 0) return;
  const int g0 = f0 / D, nh = (f1 - 1) / D - g0 + 1;
  const int nv = nsg * chunk, nm = nsg * nh;  // value words; (m, l) pairs (nm <= 2 nsg, or <= G * G)
  uint64_t vw[NV];
  bool vs[NV];
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    vw[k] = 0ull;
    vs[k] = tid + k * kThreads >= nv;
  }
  u32x4 mw = u32x4{0u, 0u, 0u, 0u};
  bool ms = tid >= nm;
  auto issue = [&]() {
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      if (!vs[k]) {
        const int idx = tid + k * kThreads, x = idx / chunk, f = f0 + idx % chunk;
        vw[k] = load_dev(grec + (size_t)x * RW + (f / D) * PD + f % D);
      }
    }
    if (!ms) {
      const int x = tid / nh, g = g0 + tid % nh;
      mw = load_dev16(grec + (size_t)x * RW + g * PD + D);
    }
  };
  auto test = [&]() -> bool {
    bool all = true;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      vs[k] = vs[k] || (uint32_t)(vw[k] >> 32) == tag;
      all = all && vs[k];
    }
    ms = ms || (mw.y == tag && mw.w == tag);
    return __ballot(!(all && ms)) == 0ull;
  };
  issue();
  if (!test()) {
    uint32_t spins = 0;
    while (true) {
      __builtin_amdgcn_s_sleep(4);
      if (++spins > kSpinLimit) {
        if (lane == 0) atomicOr(p.ws.err, kErrSpinTimeout);
        break;
      }
      issue();
      if (test()) break;
    }
  }
#pragma unroll
  for (int k = 0; k < NV; ++k)
    if (tid + k * kThreads < nv) vals[tid + k * kThreads] = __uint_as_float((uint32_t)vw[k]);
  if (tid < nm) xml[tid] = make_float2(__uint_as_float(mw.x), __uint_as_float(mw.z));
  __syncthreads();
  // per head: the maximum over the splits, each split's scale e^(m_x - M) and
  // the denominator (lanes hold splits lane and lane + 64)
  for (int gi = w; gi < nh; gi += kWaves) {
    float mx[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int x = lane + 64 * c;
      mx[c] = x < nsg ? xml[x * nh + gi].x : -INFINITY;
    }
    const float M = wave_max(fmaxf(mx[0], mx[1]));
    float part = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int x = lane + 64 * c;
      if (x < nsg) {
        const float sc = mx[c] == -INFINITY ? 0.f : expf(mx[c] - M);
        scl[x * nh + gi] = sc;
        part = fmaf(xml[x * nh + gi].y, sc, part);
      }
    }
    const float dsum = wave_sum(part);
    if (lane == 0) den[gi] = dsum;
  }
  __syncthreads();
  for (int fo = tid; fo < chunk; fo += kThreads) {
    const int gi = (f0 + fo) / D - g0;
    float num = 0.f;
    for (int x = 0; x < nsg; ++x) num = fmaf(vals[x * chunk + fo], scl[x * nh + gi], num);
    outp[f0 + fo] = num / den[gi];
  }
}

// X: every item has its own resident workgroup (grid = items) and the splits
// of a group merge by exchange; else workgroups take items in turn and the
// last split of a group to arrive merges its records.
template <int D, int G, bool X>
__global__ __launch_bounds__(kThreads) void dense_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = (float*)smem;  // [kWaves][G][D] the waves' accumulators, then the merge's per-split scales
  __shared__ DenseShared sh;
  __shared__ float2 xml[X ? kThreads : 1];  // exchange: (m, l) of the splits
  __shared__ float xscl[X ? kThreads : 1];  // exchange: e^(m - M) of the splits
  constexpr int PD = D + 2;  // partial record: acc[D], m, l
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int item = blockIdx.x;
  // Launch tag of the exchanged records (X): the launch count is the sum of
  // the kLaunchCounters launch counters, shared with the sampling kernel, and
  // every tagged launch adds exactly kLaunchUnit to it (workgroup 0 adds
  // kLaunchUnit - (grid - 1) to counter 0, workgroup x adds 1 to counter
  // x mod kLaunchCounters, each after its own reads of the counters have
  // returned).  The sum a workgroup reads is then at least L kLaunchUnit and
  // lacks its own add, so all workgroups of launch L derive the same tag, and
  // no record of an earlier launch carries it.
  uint64_t lc = 0ull;  // wave 0, lane i < kLaunchCounters: counter i as read
  if constexpr (X) {
    if (tid < kLaunchCounters) lc = load_dev(p.ws.launches + tid * kLaunchStride);
  }
  auto take_tag = [&]() {  // wave 0
    uint64_t c = tid < kLaunchCounters ? lc : 0ull;
    asm volatile("" : "+v"(c));
    uint64_t sum = 0ull;
#pragma unroll
    for (int i = 0; i < kLaunchCounters; ++i)
      sum += ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(c >> 32), i) << 32) |
             (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)c, i);
    if (tid == 0) {
      const uint32_t t = (uint32_t)(sum / kLaunchUnit) + 1u;
      sh.epoch = t == 0u ? 1u : t;
    }
  };

  while (item < p.total_items) {
    const int group = item / p.ns, s = item % p.ns;
    const int b = group / p.Hkv, hk = group % p.Hkv, h0 = hk * G;
    float* outp = p.out + (size_t)(b * p.Hq + h0) * D;
    // The length is a scalar read (it does not change during the kernel).  On
    // the resident grid (X), where every item starts with the launch, the
    // split's first K and V rows are requested before the length is used:
    // they need only the item's place and the K block's row count.  Items
    // taken in turn request them after it, and not at all for a split past
    // the sequence's end (a ragged batch has many).
    const int n = *(const __attribute__((address_space(4))) int32_t*)(p.n_k + b);
    const int k0 = s * p.split;
    DenseBuf<D, G> first;
    if constexpr (X) dense_issue<D, G>(p, b, hk, k0, first, 0, min(p.split, p.max_n_k - k0));
    const bool valid = n >= 1 && n <= p.max_n_k;
    const int nsg = valid ? (n + p.split - 1) / p.split : 0;

    if (!valid) {
      if constexpr (X) dense_drop<D, G>(first);
      if (s == 0)
        for (int i = tid; i < G * D; i += kThreads) outp[i] = __builtin_nanf("");
      if (X && w == 0) take_tag();
    } else if (s >= nsg) {
      if constexpr (X) dense_drop<D, G>(first);
      if (X && w == 0) take_tag();
    } else if (X) {
      const int len = min(p.split, n - k0);
      split_pass<D, G>(p, b, hk, k0, len, red, sh, first, true);
      if (w == 0) take_tag();
      __syncthreads();
      uint64_t* grec = p.ws.xrec + (size_t)group * p.ns * G * PD;
      finish_split<D, G>(red, sh, nsg == 1 ? kOutput : kTaggedRecord, nullptr, grec + (size_t)s * G * PD, sh.epoch,
                         outp);
      if (nsg > 1) {
        __syncthreads();  // the accumulator area is reused for the merge
        exchange_merge<D, G>(p, grec, s, nsg, sh.epoch, red, xml, xscl, sh.den, outp);
      }
    } else {
      const int len = min(p.split, n - k0);
      dense_issue<D, G>(p, b, hk, k0, first, 0, len);
      split_pass<D, G>(p, b, hk, k0, len, red, sh, first, false);
      __syncthreads();
      finish_split<D, G>(red, sh, kFloatRecord, p.ws.partial + (size_t)(group * p.ns + s) * G * PD, nullptr, 0u,
                         nullptr);
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

    if constexpr (X) {
      // this workgroup's share of the launch count (its counter reads have
      // returned: the tag was derived from them)
      const uint64_t my_add = blockIdx.x == 0 ? kLaunchUnit - (uint64_t)(p.grid - 1) : 1ull;
      if (tid == 0) atomic_add_noret(p.ws.launches + (blockIdx.x % kLaunchCounters) * kLaunchStride,
                                     lc == ~0ull ? 0ull : my_add);
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

template <int D, int G, bool X>
int capacity_t() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  auto fn = dense_kernel<D, G, X>;
  const size_t lds = DenseLds<D, G>::bytes;
  (void)hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess) return 0;
  return per_cu * cus;
}

template <int D, int G>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const size_t lds = DenseLds<D, G>::bytes;
  if (p.exch)
    hipLaunchKernelGGL((dense_kernel<D, G, true>), dim3(p.grid), dim3(kThreads), lds, stream, p);
  else
    hipLaunchKernelGGL((dense_kernel<D, G, false>), dim3(p.grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

// The smaller of the two variants' resident capacities, so that a grid
// within it is resident with either.
int dense_capacity(int D, int G) {
#define SANTA_CASE(DD, GG) \
  if (D == DD && G == GG) return std::min(capacity_t<DD, GG, false>(), capacity_t<DD, GG, true>());
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
