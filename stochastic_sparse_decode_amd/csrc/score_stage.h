// Score stage shared by the SANTA and dense decode kernels: row-major fp16 K
// streamed once with 16-byte loads; G query heads of a KV head scored per read.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace santa {

constexpr int kPer = kSplit / 64;                // CDF elements per lane in the scan
constexpr int kPad = kSplit + kSplit / 16;       // padded LDS row of one head's CDF
__device__ __forceinline__ int lidx(int j) { return j + (j >> 4); }  // bank-spread index

template <int D, int G>
struct Geo {
  static constexpr int LPR = D / 8;        // lanes per key row (16 B each)
  static constexpr int RPW = 64 / LPR;     // key rows per wave-wide load
  static constexpr int U = LPR / G;        // wave-wide loads per reduction block
  static constexpr int BR = U * RPW;       // key rows per block
  static constexpr int NB = (16 / U) > 0 ? (16 / U) : 1;   // blocks in flight per wave
  static constexpr int ROWS_IT = NB * kWaves * BR;          // rows per workgroup iteration
  static_assert(U * G == LPR, "group size must divide the row width");
};

// ---------------------------------------------------------------------------
// Score stage, row-major K: rows of D fp16 streamed with 16-byte loads, LPR
// lanes per row, U rows per lane per block so that the U*G partial dot
// products of a lane reduce-scatter to exactly one (row, head) score per lane.
// ---------------------------------------------------------------------------
template <int D, int G>
__device__ __forceinline__ void score_rowmajor(const DecodeParams& p, int b, int hk, int k0, int len,
                                               float* cdf, float* mx) {
  using Gm = Geo<D, G>;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane / Gm::LPR, c = lane % Gm::LPR;
  const _Float16* Kb = (const _Float16*)p.K + ((size_t)(b * p.Hkv + hk) * p.max_n_k + k0) * D;
  const _Float16* qb = (const _Float16*)p.q + (size_t)(b * p.Hq + hk * G) * D;
  uint4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qv[g] = *(const uint4*)(qb + g * D + c * 8);

  const int my_u = c / G, my_g = c % G;
  float* scores_out = p.scores_out ? p.scores_out + (size_t)(b * p.Hq + hk * G + my_g) * p.max_n_k + k0 : nullptr;
  float m_run = -INFINITY;

  uint4 cur[Gm::NB][Gm::U], nxt[Gm::NB][Gm::U];
  auto issue = [&](uint4 (&buf)[Gm::NB][Gm::U], int base) {
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb)
#pragma unroll
      for (int u = 0; u < Gm::U; ++u) {
        const int row = base + (nb * kWaves + w) * Gm::BR + u * Gm::RPW + r;
        buf[nb][u] = row < len ? load_nt((const uint4*)(Kb + (size_t)row * D + c * 8)) : make_uint4(0, 0, 0, 0);
      }
  };
  issue(cur, 0);
  for (int base = 0; base < len; base += Gm::ROWS_IT) {
    const int nbase = base + Gm::ROWS_IT;
    if (nbase < len) issue(nxt, nbase);
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb) {
      float v[Gm::LPR];
#pragma unroll
      for (int u = 0; u < Gm::U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) v[u * G + g] = dot8(cur[nb][u], qv[g]);
      row_reduce_scatter<Gm::LPR>(v, lane);
      const int row = base + (nb * kWaves + w) * Gm::BR + my_u * Gm::RPW + r;
      if (row < len) {
        const float s = v[0] * p.scale;
        cdf[my_g * kPad + lidx(row)] = s;
        m_run = fmaxf(m_run, s);
        if (scores_out) scores_out[row] = s;
      }
    }
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb)
#pragma unroll
      for (int u = 0; u < Gm::U; ++u) cur[nb][u] = nxt[nb][u];
  }
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = (g == my_g) ? m_run : -INFINITY;
}

}  // namespace santa
