// Score stage shared by the SANTA and dense decode kernels: row-major fp16 K
// streamed once with 16-byte loads; G query heads of a KV head scored per read.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace santa {

// LDS row of one head's scores for a split of SPLIT keys: index lidx(j) =
// j + j/16 spreads a lane's consecutive keys over the banks; the row also has
// room past its keys for one spare list slot per lane (SPLIT + lane), and its
// length is 16 mod 32 banks so that the heads' rows start on different banks.
template <int SPLIT>
constexpr int pad_of() { return SPLIT + 64 + 16; }
__device__ __forceinline__ int lidx(int j) { return j + (j >> 4); }  // bank-spread index
static_assert(pad_of<1024>() % 32 == 16 && pad_of<512>() % 32 == 16, "row length 16 mod 32 banks");

// LB = wave-wide 16-byte loads per register buffer (two buffers in flight)
template <int D, int G, int LB = 16, int SPLIT = kSplit>
struct Geo {
  static constexpr int LPR = D / 8;        // lanes per key row (16 B each)
  static constexpr int RPW = 64 / LPR;     // key rows per wave-wide load
  static constexpr int U = LPR / G;        // wave-wide loads per reduction block
  static constexpr int BR = U * RPW;       // key rows per block
  static constexpr int NB = (LB / U) > 0 ? (LB / U) : 1;   // blocks per buffer
  static constexpr int ROWS_IT = NB * kWaves * BR;          // rows per workgroup iteration
  static_assert(U * G == LPR, "group size must divide the row width");
  static_assert(SPLIT % ROWS_IT == 0, "an iteration never crosses the split end");
};

// ---------------------------------------------------------------------------
// Score stage, row-major K: rows of D fp16 streamed with 16-byte loads, LPR
// lanes per row, U rows per lane per block so that the U*G partial dot
// products of a lane reduce-scatter to exactly one (row, head) score per lane.
// ---------------------------------------------------------------------------
template <int D, int G, int LB = 16, int SPLIT = kSplit>
struct RowScore {
  using Gm = Geo<D, G, LB, SPLIT>;
  static constexpr int kPad = pad_of<SPLIT>();
  // A split is always streamed in NIT = SPLIT / ROWS_IT fully unrolled
  // iterations with two register buffers: the loads of iteration i+1 are in
  // flight while iteration i is reduced.  Loads are unconditional (rows past
  // the split's end re-read its last row, an L1 hit) so that the compiler
  // counts outstanding loads exactly and never waits for the prefetch.
  static constexpr int NIT = SPLIT / Gm::ROWS_IT;
  uint4 buf[2][Gm::NB][Gm::U];
  uint4 qv[G];
  const _Float16* Kb;
  int lane, w, r, c;

  __device__ __forceinline__ void issue(int slot, int base, int lim) {
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb)
#pragma unroll
      for (int u = 0; u < Gm::U; ++u) {
        const int row = min(base + (nb * kWaves + w) * Gm::BR + u * Gm::RPW + r, lim - 1);
        buf[slot][nb][u] = load_nt((const uint4*)(Kb + (size_t)row * D + c * 8));
      }
  }
  // The query and the first iteration's rows, clamped to the first `lim`
  // rows of the split.  lim may exceed the split's valid length, up to the
  // rows the K block holds (max_n_k - k0): the first loads can then go out
  // before the sequence length has arrived; rows past the length are scored
  // into LDS slots nothing reads and are left out of the maximum.
  __device__ __forceinline__ void begin(const DecodeParams& p, int b, int hk, int k0, int lim) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    w = tid >> 6;
    r = lane / Gm::LPR;
    c = lane % Gm::LPR;
    Kb = (const _Float16*)p.K + ((size_t)(b * p.Hkv + hk) * p.max_n_k + k0) * D;
    const _Float16* qb = (const _Float16*)p.q + (size_t)(b * p.Hq + hk * G) * D;
#pragma unroll
    for (int g = 0; g < G; ++g) qv[g] = *(const uint4*)(qb + g * D + c * 8);
    issue(0, 0, lim);
  }
  // For an item found to have nothing to score after begin(): the first
  // rows are taken as used (and waited for) on that path only, so that the
  // compiler issues them before it tests the item, not after.
  __device__ __forceinline__ void drop() {
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb)
#pragma unroll
      for (int u = 0; u < Gm::U; ++u) asm volatile("" ::"v"(buf[0][nb][u].x));
  }
  // The rest of the stage for a split of `len` valid keys.
  __device__ __forceinline__ void run(const DecodeParams& p, int len, float* cdf, float* mx) {
    const int my_u = c / G, my_g = c % G;
    float m_run = -INFINITY;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int base = it * Gm::ROWS_IT;
      if (it + 1 < NIT) issue((it + 1) & 1, base + Gm::ROWS_IT, len);
#pragma unroll
      for (int nb = 0; nb < Gm::NB; ++nb) {
        float v[Gm::LPR];
#pragma unroll
        for (int u = 0; u < Gm::U; ++u)
#pragma unroll
          for (int g = 0; g < G; ++g) v[u * G + g] = dot8(buf[it & 1][nb][u], qv[g]);
        row_reduce_scatter<Gm::LPR>(v, lane);
        // rows < SPLIT always; rows >= len land in unused LDS slots
        const int row = base + (nb * kWaves + w) * Gm::BR + my_u * Gm::RPW + r;
        const float sc = v[0] * p.scale;
        cdf[my_g * kPad + lidx(row)] = sc;
        m_run = fmaxf(m_run, row < len ? sc : -INFINITY);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) mx[g] = (g == my_g) ? m_run : -INFINITY;
  }
};

template <int D, int G, int LB = 16, int SPLIT = kSplit>
__device__ __forceinline__ void score_rowmajor(const DecodeParams& p, int b, int hk, int k0, int len,
                                               float* cdf, float* mx) {
  RowScore<D, G, LB, SPLIT> rs;
  rs.begin(p, b, hk, k0, len);
  rs.run(p, len, cdf, mx);
}

// The same stage for a paged (block table) cache: row_ptr(j) points at key
// row j (0 <= j < len) of the split.  (The contiguous stage above keeps its
// own copy: routing it through a row-pointer functor made the compiler
// schedule its loads worse.)
template <int D, int G, int LB, typename RowPtr, int SPLIT = kSplit>
__device__ __forceinline__ void score_rowmajor_rows(const DecodeParams& p, int b, int hk, int len, float* cdf,
                                                    float* mx, const RowPtr& row_ptr) {
  using Gm = Geo<D, G, LB, SPLIT>;
  constexpr int kPad = pad_of<SPLIT>();
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane / Gm::LPR, c = lane % Gm::LPR;
  const _Float16* qb = (const _Float16*)p.q + (size_t)(b * p.Hq + hk * G) * D;
  uint4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qv[g] = *(const uint4*)(qb + g * D + c * 8);

  const int my_u = c / G, my_g = c % G;
  float m_run = -INFINITY;

  // A split is always streamed in NIT = SPLIT / ROWS_IT fully unrolled
  // iterations with two register buffers: the loads of iteration i+1 are in
  // flight while iteration i is reduced.  Loads are unconditional (rows past
  // the split's end re-read its last row, an L1 hit) so that the compiler
  // counts outstanding loads exactly and never waits for the prefetch.
  constexpr int NIT = SPLIT / Gm::ROWS_IT;
  uint4 buf[2][Gm::NB][Gm::U];
  auto issue = [&](uint4 (&bb)[Gm::NB][Gm::U], int base) {
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb)
#pragma unroll
      for (int u = 0; u < Gm::U; ++u) {
        const int row = min(base + (nb * kWaves + w) * Gm::BR + u * Gm::RPW + r, len - 1);
        bb[nb][u] = load_nt((const uint4*)(row_ptr(row) + c * 8));
      }
  };
  issue(buf[0], 0);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int base = it * Gm::ROWS_IT;
    if (it + 1 < NIT) issue(buf[(it + 1) & 1], base + Gm::ROWS_IT);
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb) {
      float v[Gm::LPR];
#pragma unroll
      for (int u = 0; u < Gm::U; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) v[u * G + g] = dot8(buf[it & 1][nb][u], qv[g]);
      row_reduce_scatter<Gm::LPR>(v, lane);
      // rows < SPLIT always; rows >= len land in unused LDS slots
      const int row = base + (nb * kWaves + w) * Gm::BR + my_u * Gm::RPW + r;
      const float s = v[0] * p.scale;
      cdf[my_g * kPad + lidx(row)] = s;
      m_run = fmaxf(m_run, row < len ? s : -INFINITY);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = (g == my_g) ? m_run : -INFINITY;
}

// ---------------------------------------------------------------------------
// Score stage, fp8 key cache: rows of D bytes (OCP E4M3), 16 bytes = 16
// features per lane, LPR = D / 16 lanes per row.  Each 16-byte piece becomes
// eight fp16 pairs (the E4M3 -> fp16 conversion is exact) that are dotted
// with the query's fp16 pairs (v_dot2_f32_f16, fp32 accumulate); the sum is
// scaled by scale * k_scale[b, h_kv] once.  Same schedule as the fp16 stage.
// ---------------------------------------------------------------------------
template <int D, int G, int LB = 16, int SPLIT = kSplit>
struct GeoF8 {
  static constexpr int LPR = D / 16;       // lanes per key row (16 B each)
  static constexpr int RPW = 64 / LPR;     // key rows per wave-wide load
  static constexpr int U = LPR / G;        // wave-wide loads per reduction block
  static constexpr int BR = U * RPW;       // key rows per block
  static constexpr int NB = (LB / U) > 0 ? (LB / U) : 1;   // blocks per buffer
  static constexpr int ROWS_IT = NB * kWaves * BR;          // rows per workgroup iteration
  static_assert(U >= 1 && U * G == LPR, "group size must divide the row width");
  static_assert(SPLIT % ROWS_IT == 0, "an iteration never crosses the split end");
};

template <int D, int G>
constexpr bool fp8_supported() { return G <= D / 16; }

template <int D, int G, int LB = 16, int SPLIT = kSplit>
struct RowScoreF8 {
  using Gm = GeoF8<D, G, LB, SPLIT>;
  static constexpr int kPad = pad_of<SPLIT>();
  static constexpr int NIT = SPLIT / Gm::ROWS_IT;
  uint4 buf[2][Gm::NB][Gm::U];
  uint4 qv[G][2];  // features c*16 .. c*16+15 of each head, as fp16 pairs
  const uint8_t* Kb;
  float sc;
  int lane, w, r, c;

  __device__ __forceinline__ void issue(int slot, int base, int lim) {
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb)
#pragma unroll
      for (int u = 0; u < Gm::U; ++u) {
        const int row = min(base + (nb * kWaves + w) * Gm::BR + u * Gm::RPW + r, lim - 1);
        buf[slot][nb][u] = load_nt((const uint4*)(Kb + (size_t)row * D + c * 16));
      }
  }
  // The query, the key scale and the first iteration's rows, clamped to the
  // first `lim` rows of the split (as RowScore::begin).
  __device__ __forceinline__ void begin(const DecodeParams& p, int b, int hk, int k0, int lim) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    w = tid >> 6;
    r = lane / Gm::LPR;
    c = lane % Gm::LPR;
    Kb = (const uint8_t*)p.K + ((size_t)(b * p.Hkv + hk) * p.max_n_k + k0) * D;
    const _Float16* qb = (const _Float16*)p.q + (size_t)(b * p.Hq + hk * G) * D;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      qv[g][0] = *(const uint4*)(qb + g * D + c * 16);
      qv[g][1] = *(const uint4*)(qb + g * D + c * 16 + 8);
    }
    sc = p.scale * p.k_scale[b * p.Hkv + hk];
    issue(0, 0, lim);
  }
  __device__ __forceinline__ void drop() {
#pragma unroll
    for (int nb = 0; nb < Gm::NB; ++nb)
#pragma unroll
      for (int u = 0; u < Gm::U; ++u) asm volatile("" ::"v"(buf[0][nb][u].x));
  }
  __device__ __forceinline__ void run(const DecodeParams& p, int len, float* cdf, float* mx) {
    const int my_u = c / G, my_g = c % G;
    float m_run = -INFINITY;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int base = it * Gm::ROWS_IT;
      if (it + 1 < NIT) issue((it + 1) & 1, base + Gm::ROWS_IT, len);
#pragma unroll
      for (int nb = 0; nb < Gm::NB; ++nb) {
        float v[Gm::LPR];
#pragma unroll
        for (int u = 0; u < Gm::U; ++u) {
          // fp16 pairs of features (2m, 2m+1) of the lane's 16
          uint32_t kh[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t wd = word_of(buf[it & 1][nb][u], i);
            kh[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd, 1.0f, false));
            kh[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd, 1.0f, true));
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m)
              acc = __builtin_amdgcn_fdot2(as_h2(kh[m]), as_h2(word_of(qv[g][m >> 2], m & 3)), acc, false);
            v[u * G + g] = acc;
          }
        }
        row_reduce_scatter<Gm::LPR>(v, lane);
        // rows < SPLIT always; rows >= len land in unused LDS slots
        const int row = base + (nb * kWaves + w) * Gm::BR + my_u * Gm::RPW + r;
        const float s = v[0] * sc;
        cdf[my_g * kPad + lidx(row)] = s;
        m_run = fmaxf(m_run, row < len ? s : -INFINITY);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) mx[g] = (g == my_g) ? m_run : -INFINITY;
  }
};

template <int D, int G, int LB = 16, int SPLIT = kSplit>
__device__ __forceinline__ void score_rowmajor_f8(const DecodeParams& p, int b, int hk, int k0, int len,
                                                  float* cdf, float* mx) {
  RowScoreF8<D, G, LB, SPLIT> rs;
  rs.begin(p, b, hk, k0, len);
  rs.run(p, len, cdf, mx);
}

// Copy the split's scores from LDS to scores_out (debug output), coalesced.
template <int G, int SPLIT = kSplit>
__device__ __forceinline__ void write_scores(const DecodeParams& p, int b, int hk, int k0, int len, const float* cdf) {
  constexpr int kPad = pad_of<SPLIT>();
  if (!p.scores_out) return;
  for (int i = threadIdx.x; i < G * len; i += kThreads) {
    const int g = i / len, j = i % len;
    p.scores_out[(size_t)(b * p.Hq + hk * G + g) * p.max_n_k + k0 + j] = cdf[g * kPad + lidx(j)];
  }
}

}  // namespace santa
