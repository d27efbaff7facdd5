// SANTA stochastic sparse decode step: one fused, persistent kernel.
//
// Method: "Stochastic Sparse Attention for Memory-Bound Inference"
// (arXiv 2605.01910), abstract.  Every key is scored (the score stage still
// reads all of K); S key indices are drawn from the post-softmax distribution
// by inverse-CDF sampling (i.i.d., stratified, or systematic with a single
// offset), and only those value rows are gathered and added, divided by S,
// which estimates softmax(qK^T)V without bias.  In the Bernoulli qK^T mode
// the query is replaced by a stochastic ternary vector so that only the kept
// key features are read.
//
// Work decomposition (one GPU, gfx950):
//   work item = (sequence b, KV head, split of kSplit keys).  Items of one KV
//   head ("group") are consecutive.  Each workgroup (256 threads) takes an
//   item, streams that split's K rows once with 16-byte loads, scores the G
//   query heads of the group (GQA packing: one K read serves G heads), keeps
//   the scores in LDS, turns them into a local CDF (prefix sums of
//   exp(s - local max)), publishes (local max, local sum) and waits until all
//   splits of the group have published.  From the merged statistics every
//   workgroup knows the global normaliser and its split's CDF offset, places
//   the stratum points that fall in its probability range, searches its local
//   CDF, gathers each selected value row once (adding it count times), and
//   writes a partial sum.  The last workgroup of the group to finish adds the
//   partials in split order and writes the output.
//
// Scheduling: `grid` workgroups are all resident (grid <= occupancy capacity).
// Workgroup w starts with item w; further items are taken in increasing order
// from an atomic counter.  A workgroup only waits for splits of its own group,
// all of which have been taken by running workgroups or will be taken by
// workgroups that finish earlier groups, so the waits always end as long as a
// group has no more splits than there are workgroups.  Every wait is bounded
// (kSpinLimit polls); a timeout sets an error bit instead of hanging.
#include "device_common.h"
#include "launch.h"
#include "score_stage.h"

namespace santa {

namespace {

template <int D, int G>
struct Lds {
  // float cdf[G][kPad]; uint32 cnt[G][kSplit]; aux (uniform bits / reduction / list)
  static constexpr size_t cdf_bytes = sizeof(float) * G * kPad;
  static constexpr size_t cnt_bytes = sizeof(uint32_t) * G * kSplit;
  static constexpr size_t uni_bytes = sizeof(uint32_t) * G * kMaxS;
  static constexpr size_t red_bytes = sizeof(float) * kWaves * G * D;
  static constexpr size_t list_bytes = sizeof(uint32_t) * kSplit;
  static constexpr size_t aux_bytes =
      uni_bytes > red_bytes ? (uni_bytes > list_bytes ? uni_bytes : list_bytes)
                            : (red_bytes > list_bytes ? red_bytes : list_bytes);
  static constexpr size_t bytes = cdf_bytes + cnt_bytes + aux_bytes;
};

struct Shared {
  float wmax[kWaves][8];
  float lsum[8];
  double Z[8], SZ[8], Olo[8], Ohi[8], rs[8], usys[8];
  int wcount[kWaves];
  int n_distinct;
  int last;
  int next_item;
  // Bernoulli mode
  float A[8];
  int nu;
};

// ---------------------------------------------------------------------------
// Score stage, Bernoulli qK^T: the ternary query keeps feature i of head g
// when u_i * A_g < |q_gi| (A_g = max_i |q_gi|, u_i shared by the group), with
// value sign(q_gi) * A_g.  K is stored as 64-key feature-major tiles, so each
// kept feature of a tile is one contiguous 128-byte row; only the union of
// the group's kept features is read, and each contributes by add/subtract.
// ---------------------------------------------------------------------------
template <int D, int G>
__device__ __forceinline__ void bernoulli_setup(const DecodeParams& p, int b, int hk, bool write_kept,
                                                Shared& sh, uint32_t* info) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const _Float16* qb = (const _Float16*)p.q + (size_t)(b * p.Hq + hk * G) * D;
  // A_g = max |q_g| : wave g-loop over features
  if (w == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a = 0.f;
      for (int i = lane; i < D; i += 64) a = fmaxf(a, fabsf((float)qb[g * D + i]));
      for (int m = 1; m < 64; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
      if (lane == 0) sh.A[g] = a;
    }
  }
  __syncthreads();
  bool any = false;
  uint32_t bits = 0;
  if (tid < D) {
    const uint4 blk = stream_block(p.seed, (uint32_t)(b * p.Hkv + hk), kTagBernoulli, (uint32_t)(tid >> 2));
    const double ub = (double)uniform_bits(word_of(blk, tid & 3));
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float qi = (float)qb[g * D + tid];
      // u * A < |q|  <=>  (x >> 8) * A < |q| * 2^24, exact in fp64
      const bool keep = ub * (double)sh.A[g] < (double)fabsf(qi) * 16777216.0;
      if (keep) bits |= (1u << (2 * g)) | ((qi < 0.f ? 1u : 0u) << (2 * g + 1));
      any |= keep;
      if (write_kept) p.kept_out[(size_t)(b * p.Hq + hk * G + g) * D + tid] = keep ? 1 : 0;
    }
  }
  // compact the union of kept features in increasing feature order
  const uint64_t bal = __ballot(any);
  const int before = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0 && w < 2) sh.wcount[w] = __popcll(bal);
  __syncthreads();
  if (any) {
    const int pos = before + (w == 1 ? sh.wcount[0] : 0);
    info[pos] = ((uint32_t)tid << 16) | bits;
  }
  if (tid == 0) sh.nu = (D > 64) ? sh.wcount[0] + sh.wcount[1] : sh.wcount[0];
  __syncthreads();
}

template <int D, int G>
__device__ __forceinline__ void score_bernoulli(const DecodeParams& p, int b, int hk, int k0, int len,
                                                float* cdf, float* mx, const Shared& sh, const uint32_t* info) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, t4 = (lane >> 3) & 3, ko = lane & 7;
  const int ti = w * 4 + t4;  // tile of this lane inside the split (16 tiles)
  const int tiles_per_head = p.max_n_k / kTile;
  // tiles past the sequence end re-read its last tile (results discarded)
  const int tile = min(k0 / kTile + ti, (k0 + len - 1) / kTile);
  const _Float16* tb = (const _Float16*)p.K + ((size_t)(b * p.Hkv + hk) * tiles_per_head + tile) * (size_t)(D * kTile);
  const int nu = sh.nu;
  float acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;

  constexpr int UNR = 8;
  const int steps = (nu + 1) / 2;
  for (int f0 = 0; f0 < steps; f0 += UNR) {
    uint4 kv[UNR];
    uint32_t inf[UNR];
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
      const int fi = 2 * (f0 + x) + half;
      const bool ok = fi < nu;
      const uint32_t e = info[ok ? fi : 0];       // nu >= 1 here
      inf[x] = ok ? e : (e & 0xffff0000u);          // past the list: keep nothing
      kv[x] = load_nt((const uint4*)(tb + (size_t)(e >> 16) * kTile + ko * 8));
    }
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
      float f[8];
      unpack8(kv[x], f);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const bool keep = (inf[x] >> (2 * g)) & 1u;
        const bool neg = (inf[x] >> (2 * g + 1)) & 1u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float t = neg ? -f[e] : f[e];
          acc[g][e] += keep ? t : 0.f;
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mx[g] = -INFINITY;
    const float sc = p.scale * sh.A[g];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float tot = acc[g][e] + __shfl_xor(acc[g][e], 32, 64);
      const int row = ti * kTile + ko * 8 + e;
      const float s = tot * sc;
      if (half == 0 && row < len) {
        cdf[g * kPad + lidx(row)] = s;
        mx[g] = fmaxf(mx[g], s);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sampling helpers.
//
// Masses are fixed-point integers in units of 2^-31 of a split's largest
// weight: w = exp(s - m) in (0, 1] becomes q = trunc(w * 2^31), the local CDF
// c_j = q_0 + ... + q_j is an exact integer (stored as an fp32 value, which
// keeps it nondecreasing), and the split masses merged across the group are
// integers too, so split offsets O_s are exact, nondecreasing and identical
// in every workgroup.  In global units the right edge of key j of split s is
// x_j = O_s + r_s c_j with r_s = exp(m_s - M); the edges are clamped to the
// split's range [O_s, O_{s+1}], so the keys of all splits tile [0, Z)
// without gaps or overlaps.  A point t selects the key whose interval holds
// t Z (the inverse CDF, with the half-open convention x_{j-1} <= t Z < x_j).
// ---------------------------------------------------------------------------
constexpr float kFix = 2147483648.0f;  // 2^31

struct PointSet {
  int mode, S;
  double SZ;           // S / Z
  double u;            // systematic offset
  const uint32_t* ub;  // stratified: 24-bit uniforms of the S strata
};

// Number of stratum points with (k + u_k) / S < x / Z (x in mass units).
// Systematic: #{k : k + u < y} = ceil(y - u); stratified: all strata below
// floor(y) plus stratum floor(y) when its uniform lies below y - floor(y).
__device__ __forceinline__ int points_below(const PointSet& ps, double x) {
  const double y = x * ps.SZ;
  if (ps.mode == 2) {
    const double v = ceil(y - ps.u);
    return v <= 0.0 ? 0 : (v >= (double)ps.S ? ps.S : (int)v);
  }
  if (!(y > 0.0)) return 0;
  const double m = floor(y);
  if (m >= (double)ps.S) return ps.S;
  const int mi = (int)m;
  return mi + ((double)ps.ub[mi] * 0x1.0p-24 < y - m ? 1 : 0);
}

// First key j in [0, len) whose right edge O + r c_j exceeds tz, else len - 1.
__device__ __forceinline__ int key_of(const float* c, int len, double O, double r, double tz) {
  int lo = 0, hi = len;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (fma(r, (double)c[lidx(mid)], O) > tz) hi = mid; else lo = mid + 1;
  }
  return lo < len ? lo : len - 1;
}

// ---------------------------------------------------------------------------
// The fused kernel.
// ---------------------------------------------------------------------------
template <int D, int G, bool BERN>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  using L = Lds<D, G>;
  float* cdf = (float*)smem;                                   // [G][kPad] scores, then local CDF
  uint32_t* cnt = (uint32_t*)(smem + L::cdf_bytes);             // [G][kSplit] points per key
  unsigned char* aux = smem + L::cdf_bytes + L::cnt_bytes;
  uint32_t* uni = (uint32_t*)aux;   // [G][kMaxS] 24-bit uniforms (stratified, i.i.d.)
  float* red = (float*)aux;         // [kWaves][G*D] gather reduction
  uint32_t* list = (uint32_t*)aux;  // [kSplit] distinct selected keys
  __shared__ Shared sh;
  __shared__ uint32_t binfo[128];   // Bernoulli kept-feature union

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int S = p.S;
  int item = blockIdx.x;

  while (item < p.total_items) {
    const int group = item / p.ns, s = item % p.ns;
    const int b = group / p.Hkv, hk = group % p.Hkv, h0 = hk * G;
    const int n = p.n_k[b];
    const bool valid = n >= 1 && n <= p.max_n_k;
    const int nsg = valid ? (n + kSplit - 1) / kSplit : 0;

    if (!valid) {
      if (s == 0) {  // invalid sequence length: NaN output, indices -1
        for (int i = tid; i < G * D; i += kThreads) p.out[(size_t)(b * p.Hq + h0) * D + i] = __builtin_nanf("");
        if (p.idx_out)
          for (int i = tid; i < G * S; i += kThreads) p.idx_out[(size_t)(b * p.Hq + h0) * S + i] = -1;
      }
    } else if (s < nsg) {
      const int k0 = s * kSplit;
      const int len = min(kSplit, n - k0);
      const bool is_last = (s == nsg - 1);
      float mx[G];

      // ---- score stage: all keys of the split, G query heads ----------------
      if constexpr (BERN) {
        bernoulli_setup<D, G>(p, b, hk, p.kept_out != nullptr && s == 0, sh, binfo);
        score_bernoulli<D, G>(p, b, hk, k0, len, cdf, mx, sh, binfo);
      } else {
        score_rowmajor<D, G>(p, b, hk, k0, len, cdf, mx);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m = wave_max_masked(mx[g], 1);
        if (lane == 0) sh.wmax[w][g] = m;
      }
      __syncthreads();
      if (p.scores_out) {
        write_scores<G>(p, b, hk, k0, len, cdf);
        __syncthreads();
      }

      // ---- local CDF in fixed point, one wave per head ----------------------
      for (int g = w; g < G; g += kWaves) {
        float m = sh.wmax[0][g];
#pragma unroll
        for (int x = 1; x < kWaves; ++x) m = fmaxf(m, sh.wmax[x][g]);
        float* cg = cdf + g * kPad;
        uint64_t run[kPer];
        uint64_t acc = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int j = lane * kPer + i;
          const uint32_t q = j < len ? (uint32_t)(expf(cg[lidx(j)] - m) * kFix) : 0u;
          acc += q;
          run[i] = acc;
        }
        const uint64_t excl = wave_incl_scan_u64(acc) - acc;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const int j = lane * kPer + i;
          if (j < len) {
            const float cv = (float)(excl + run[i]);
            cg[lidx(j)] = cv;
            if (j == len - 1) sh.lsum[g] = cv;
          }
        }
        if (lane == 0) sh.wmax[0][g] = m;
      }
      __syncthreads();

      // ---- publish (split max, split mass); the slot doubles as the flag ----
      float2* slots = p.ws.stats + (size_t)group * p.ns * G;  // [split][head]
      if (tid < G) {
        float l = sh.lsum[tid];
        if (__float_as_uint(l) == 0u) l = -0.0f;  // never publish the all-zero pattern (NaN inputs)
        store_dev(slots + s * G + tid, make_float2(sh.wmax[0][tid], l));
      }

      // while the other splits finish: uniforms of the points
      if (p.mode != 2) {
        const int nb = (S + 3) >> 2;
        const uint32_t tag = p.mode == 1 ? kTagStratified : kTagIid;
        for (int t = tid; t < G * nb; t += kThreads) {
          const int g = t / nb, kb = t % nb;
          const uint4 blk = stream_block(p.seed, (uint32_t)(b * p.Hq + h0 + g), tag, (uint32_t)kb);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kb * 4 + e < S) uni[g * kMaxS + kb * 4 + e] = uniform_bits(word_of(blk, e));
        }
        if (p.mode == 0)
          for (int i = tid; i < G * kSplit; i += kThreads) cnt[i] = 0u;
      } else if (tid < G) {
        sh.usys[tid] = uniform_f64(stream_block(p.seed, (uint32_t)(b * p.Hq + h0 + tid), kTagSystematic, 0u).x);
      }
      __syncthreads();

      // ---- wait for every split of the group, merge (one wave per head) -----
      for (int g = w; g < G; g += kWaves) {
        float2 v0 = make_float2(-INFINITY, 1.f);
        for (int c0 = 0; c0 < nsg; c0 += 64) {  // poll every chunk of 64 splits
          const int x = c0 + lane;
          uint32_t spins = 0;
          while (true) {
            const float2 v = x < nsg ? load_dev(slots + x * G + g) : make_float2(-INFINITY, 1.f);
            if (c0 == 0) v0 = v;
            if (__ballot(__float_as_uint(v.y) == 0u) == 0ull) break;  // published mass is never +0.0
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
              if (lane == 0) atomicOr(p.ws.err, kErrSpinTimeout);
              break;
            }
          }
        }
        float Mloc = -INFINITY;
        for (int c0 = 0; c0 < nsg; c0 += 64) {
          const int x = c0 + lane;
          const float2 v = c0 == 0 ? v0 : (x < nsg ? load_dev(slots + x * G + g) : make_float2(-INFINITY, 1.f));
          Mloc = fmaxf(Mloc, v.x);
        }
        const float M = wave_max_masked(Mloc, 1);
        uint64_t carry = 0;
        for (int c0 = 0; c0 < nsg; c0 += 64) {
          const int x = c0 + lane;
          float2 v = c0 == 0 ? v0 : (x < nsg ? load_dev(slots + x * G + g) : make_float2(-INFINITY, 0.f));
          const float r = x < nsg ? expf(v.x - M) : 0.f;
          const uint64_t Q = x < nsg ? (uint64_t)((double)v.y * (double)r) : 0ull;
          const uint64_t incl = wave_incl_scan_u64(Q) + carry;
          if (x == s) {
            sh.Olo[g] = (double)(incl - Q);
            sh.Ohi[g] = (double)incl;
            sh.rs[g] = (double)r;
          }
          carry = wave_bcast_u64(incl, 63);
        }
        if (lane == 0) {
          sh.Z[g] = (double)carry;
          sh.SZ[g] = (double)S / (double)carry;
        }
      }
      __syncthreads();

      // ---- points per key -----------------------------------------------------
      constexpr int KPT = kSplit / kThreads;
      if (p.mode != 0) {
        // stratified / systematic: the count of key j is the number of points
        // below its right edge minus the number below its left edge
        for (int g = 0; g < G; ++g) {
          const PointSet ps{p.mode, S, sh.SZ[g], sh.usys[g], uni + g * kMaxS};
          const double O = sh.Olo[g], r = sh.rs[g];
          const int Plo = points_below(ps, O);
          const int Phi = is_last ? S : points_below(ps, sh.Ohi[g]);
          const float* cg = cdf + g * kPad;
          const int j0 = tid * KPT;
          if (j0 >= len) continue;
          int prev = j0 == 0 ? Plo : min(max(points_below(ps, fma(r, (double)cg[lidx(j0 - 1)], O)), Plo), Phi);
          const size_t row = (size_t)(b * p.Hq + h0 + g);
#pragma unroll
          for (int x = 0; x < KPT; ++x) {
            const int j = j0 + x;
            if (j >= len) break;
            const int up = j == len - 1 ? Phi : min(max(points_below(ps, fma(r, (double)cg[lidx(j)], O)), Plo), Phi);
            cnt[g * kSplit + j] = (uint32_t)(up - prev);
            if (p.idx_out)
              for (int k = prev; k < up; ++k) p.idx_out[row * S + k] = k0 + j;
            prev = up;
          }
        }
      } else {
        // i.i.d.: every point is tested against this split's range and
        // searched in the local CDF
        for (int pi = tid; pi < G * S; pi += kThreads) {
          const int g = pi / S, k = pi % S;
          const uint32_t ub = uni[g * kMaxS + k];
          const double tz = (double)ub * 0x1.0p-24 * sh.Z[g];
          if (tz < sh.Olo[g] || (!is_last && tz >= sh.Ohi[g])) continue;
          const int j = key_of(cdf + g * kPad, len, sh.Olo[g], sh.rs[g], tz);
          atomicAdd(&cnt[g * kSplit + j], 1u);
          if (p.idx_out) {  // position in the sorted list: rank among the S uniforms, ties by stream index
            const uint32_t* ug = uni + g * kMaxS;
            int rk = 0;
            for (int x = 0; x < S; ++x) rk += (ug[x] < ub) || (ug[x] == ub && x < k);
            p.idx_out[(size_t)(b * p.Hq + h0 + g) * S + rk] = k0 + j;
          }
        }
      }
      __syncthreads();

      // ---- distinct selected keys, in key order ------------------------------
      int flags = 0, nf = 0;
#pragma unroll
      for (int x = 0; x < KPT; ++x) {
        const int j = tid * KPT + x;
        bool any = false;
#pragma unroll
        for (int g = 0; g < G; ++g) any |= cnt[g * kSplit + j] != 0u;
        if (any && j < len) {
          flags |= 1 << x;
          ++nf;
        }
      }
      const int incl_n = wave_incl_scan_i32(nf, lane);
      if (lane == 63) sh.wcount[w] = incl_n;
      __syncthreads();
      int base = incl_n - nf;
      for (int x = 0; x < w; ++x) base += sh.wcount[x];
      if (tid == kThreads - 1) {
        int tot = 0;
        for (int x = 0; x < kWaves; ++x) tot += sh.wcount[x];
        sh.n_distinct = tot;
      }
#pragma unroll
      for (int x = 0; x < KPT; ++x)
        if (flags & (1 << x)) list[base++] = (uint32_t)(tid * KPT + x);
      __syncthreads();

      // ---- gather-add: each distinct row once, added `count` times ---------
      {
        constexpr int LPR = D / 8, RPW = 64 / LPR;
        const int r = lane / LPR, c = lane % LPR;
        const _Float16* Vb = (const _Float16*)p.V + ((size_t)(b * p.Hkv + hk) * p.max_n_k + k0) * D;
        float acc[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
        const int nd = sh.n_distinct;
        for (int i = w * RPW + r; i < nd; i += kWaves * RPW) {
          const int j = (int)list[i];
          float f[8];
          unpack8(*(const uint4*)(Vb + (size_t)j * D + c * 8), f);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float cf = (float)cnt[g * kSplit + j];  // count * v is exact (count <= 1024)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(cf, f[e], acc[g][e]);
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            for (int m = LPR; m < 64; m <<= 1) acc[g][e] += __shfl_xor(acc[g][e], m, 64);
        __syncthreads();  // `list` aliases `red`
        if (r == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[w * G * D + g * D + c * 8 + e] = acc[g][e];
        }
      }
      __syncthreads();
      float* part = p.ws.partial + (size_t)(group * p.ns + s) * G * D;
      for (int i = tid; i < G * D; i += kThreads) {
        float v = red[i];
#pragma unroll
        for (int x = 1; x < kWaves; ++x) v += red[x * G * D + i];
        store_dev(part + i, v);
      }
      wait_memory();
      __syncthreads();
      if (tid == 0) sh.last = atomic_add_dev(p.ws.bar_done + group, 1u) == (uint32_t)(nsg - 1);
      __syncthreads();

      // ---- last split of the group: add partials in split order -----------
      if (sh.last) {
        const float* gp = p.ws.partial + (size_t)group * p.ns * G * D;
        constexpr int OPT = (G * D + kThreads - 1) / kThreads;
        constexpr int CH = 32;  // splits loaded at once
        float sum[OPT];
#pragma unroll
        for (int o = 0; o < OPT; ++o) sum[o] = 0.f;
        for (int x0 = 0; x0 < nsg; x0 += CH) {
          float t[OPT][CH];
#pragma unroll
          for (int o = 0; o < OPT; ++o)
#pragma unroll
            for (int u = 0; u < CH; ++u) {
              const int i = min(tid + o * kThreads, G * D - 1);
              t[o][u] = load_dev(gp + (size_t)min(x0 + u, nsg - 1) * G * D + i);
            }
#pragma unroll
          for (int o = 0; o < OPT; ++o)
#pragma unroll
            for (int u = 0; u < CH; ++u) sum[o] += x0 + u < nsg ? t[o][u] : 0.f;
        }
#pragma unroll
        for (int o = 0; o < OPT; ++o) {
          const int i = tid + o * kThreads;
          if (i < G * D) p.out[(size_t)(b * p.Hq + h0) * D + i] = sum[o] / (float)S;
        }
        // leave the group's flags at zero for the next launch
        for (int i = tid; i < nsg * G; i += kThreads) store_dev(slots + i, make_float2(0.f, 0.f));
        if (tid == 0) store_dev(p.ws.bar_done + group, 0u);
      }
    }

    // ---- next work item ----------------------------------------------------
    if (p.grid >= p.total_items) break;
    __syncthreads();
    if (tid == 0) {
      const uint32_t t = atomic_add_dev(p.ws.work_ctr, 1u);
      sh.next_item = p.grid + (int)t;
      if (t == (uint32_t)(p.total_items - 1)) store_dev(p.ws.work_ctr, 0u);  // last grab of the launch
    }
    __syncthreads();
    item = sh.next_item;
  }
}

template <int D, int G, bool BERN>
size_t lds_bytes() { return Lds<D, G>::bytes; }

template <int D, int G, bool BERN>
int capacity_t() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  auto fn = decode_kernel<D, G, BERN>;
  const size_t lds = lds_bytes<D, G, BERN>();
  (void)hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess) return 0;
  return per_cu * cus;
}

template <int D, int G, bool BERN>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const size_t lds = lds_bytes<D, G, BERN>();
  hipLaunchKernelGGL((decode_kernel<D, G, BERN>), dim3(p.grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <bool BERN>
hipError_t dispatch(const DecodeParams& p, hipStream_t stream) {
#define SANTA_CASE(DD, GG) \
  if (p.D == DD && p.G == GG) return launch_t<DD, GG, BERN>(p, stream);
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return hipErrorInvalidValue;
}

template <bool BERN>
int capacity(int D, int G) {
#define SANTA_CASE(DD, GG) \
  if (D == DD && G == GG) return capacity_t<DD, GG, BERN>();
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return 0;
}

}  // namespace

int decode_capacity(int D, int G, bool bernoulli) { return bernoulli ? capacity<true>(D, G) : capacity<false>(D, G); }

hipError_t launch_decode(const DecodeParams& p, bool bernoulli, hipStream_t stream) {
  return bernoulli ? dispatch<true>(p, stream) : dispatch<false>(p, stream);
}

}  // namespace santa
