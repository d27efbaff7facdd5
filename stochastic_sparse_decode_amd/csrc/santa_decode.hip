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
  double Z[8], Olo[8], Ohi[8], rs[8], usys[8];
  int klo[8], ncand[8], npts[8];
  uint32_t bits[kSplit / 32];  // keys of the split chosen by any head
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
// The local CDF is accumulated in doubles holding integers (exact sums).
// ---------------------------------------------------------------------------
constexpr float kFix = 2147483648.0f;  // 2^31

// First key j in [0, len) whose local CDF value c_j exceeds tau, else
// len - 1.  tau = (t Z - O_s) / r_s is the point in the split's own units, so
// the probes are plain fp32 compares; a monotone rule inside the split keeps
// the keys of all splits a partition of [0, Z).  Four-way search: three
// independent probes per round (one LDS latency), then the last <= 4
// candidates counted at once.
__device__ __forceinline__ int key_of(const float* c, int len, float tau) {
  int lo = 0, hi = len;  // the answer lies in [lo, hi]
  while (hi - lo > 4) {
    const int q = (hi - lo) >> 2;
    const int m1 = lo + q, m2 = lo + 2 * q, m3 = lo + 3 * q;
    const bool b1 = c[lidx(m1)] > tau;
    const bool b2 = c[lidx(m2)] > tau;
    const bool b3 = c[lidx(m3)] > tau;
    lo = b1 ? lo : (b2 ? m1 + 1 : (b3 ? m2 + 1 : m3 + 1));
    hi = b1 ? m1 : (b2 ? m2 : (b3 ? m3 : hi));
  }
  int below = 0;  // values <= tau among the last candidates (the values are nondecreasing)
#pragma unroll
  for (int x = 0; x < 4; ++x) below += (lo + x < hi && c[lidx(min(lo + x, len - 1))] <= tau) ? 1 : 0;
  const int j = lo + below;
  return j < len ? j : len - 1;
}

// ---------------------------------------------------------------------------
// The fused kernel.
// ---------------------------------------------------------------------------
// OCC = workgroups per CU the register budget is sized for: 1 when every work
// item has its own workgroup (no item waits behind another), 2 when
// workgroups take several items in turn, so that one workgroup streams K
// while the other is in the latency-bound sampling tail of its item.
template <int D, int G, bool BERN, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void decode_kernel(DecodeParams p) {
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
  // Launch tag of the statistics slots: the workspace's launch number + 1.
  // Every workgroup reads the number before any workgroup of this launch can
  // advance it (that happens when the last one exits), so all agree, and a
  // slot left by an earlier launch (or an earlier replay of a captured graph)
  // never carries this tag.
  // (the load is issued here and first waited for when a slot is written)
  const uint32_t ep_base = load_dev(p.ws.epoch);
  auto launch_tag = [&]() -> uint32_t { return ep_base + 1u == 0u ? 1u : ep_base + 1u; };
  // Each workgroup, once its read of the launch number has completed, counts
  // itself in; the last one counted advances the number for the next launch
  // (at its exit), when every workgroup of this launch has read it.  The
  // count is taken after the first item's output adds are issued (the read
  // was consumed when the slots were written), so its round trip overlaps
  // theirs.
  uint32_t entered = 0xffffffffu;

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
      // split 0 clears the group's output rows; every split adds into them
      // only after all splits (split 0 included) have published statistics
      if (s == 0)
        for (int i = tid; i < G * D; i += kThreads) store_dev(p.out + (size_t)(b * p.Hq + h0) * D + i, 0.f);
      // per-key counts, the key bitmap and per-head point counts start at 0
      // (done here, while the first K loads are in flight)
      for (int i = tid; i < G * kSplit / 4; i += kThreads) ((uint4*)cnt)[i] = make_uint4(0, 0, 0, 0);
      if (tid < G) sh.npts[tid] = 0;
      if (tid < kSplit / 32) sh.bits[tid] = 0u;
      if (tid < G && p.mode == 2)
        sh.usys[tid] = uniform_f64(stream_block(p.seed, (uint32_t)(b * p.Hq + h0 + tid), kTagSystematic, 0u).x);

      // ---- score stage: all keys of the split, G query heads ----------------
      if constexpr (BERN) {
        bernoulli_setup<D, G>(p, b, hk, p.kept_out != nullptr && s == 0, sh, binfo);
        score_bernoulli<D, G>(p, b, hk, k0, len, cdf, mx, sh, binfo);
      } else {
        score_rowmajor<D, G>(p, b, hk, k0, len, cdf, mx);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m = wave_max(mx[g]);
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
        double run[kPer];  // integer-valued: every sum below is exact
        double acc = 0.0;
        float sv[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) sv[i] = cg[lidx(lane * kPer + i)];  // all reads issued together
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
          const double q = trunc((double)expf(sv[i] - m) * kFix);
          acc += lane * kPer + i < len ? q : 0.0;
          run[i] = acc;
        }
        const double excl = wave_incl_scan_exact(acc) - acc;
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
      // each half of a slot carries the launch tag, so a reader accepts it
      // only when both halves were written by this launch
      uint64_t* slots = p.ws.stats + (size_t)group * p.ns * G * 2;  // [split][head][2]
      if (tid < G) {
        const uint64_t tag = (uint64_t)launch_tag() << 32;
        if (s == 0) wait_memory();  // the cleared output rows are visible first
        store_dev(slots + (s * G + tid) * 2, tag | __float_as_uint(sh.wmax[0][tid]));
        store_dev(slots + (s * G + tid) * 2 + 1, tag | __float_as_uint(sh.lsum[tid]));
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
        __syncthreads();
      }

      // ---- wait for every split of the group, merge (one wave per head) -----
      const uint32_t ep = launch_tag();
      for (int g = w; g < G; g += kWaves) {
        float2 v0 = make_float2(-INFINITY, 0.f);  // (split max, split mass) of lane's split, chunk 0
        auto read_slot = [&](int x, bool& ok) -> float2 {
          const uint64_t a = load_dev(slots + (x * G + g) * 2);
          const uint64_t c = load_dev(slots + (x * G + g) * 2 + 1);
          ok = (uint32_t)(a >> 32) == ep && (uint32_t)(c >> 32) == ep;
          return make_float2(__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)c));
        };
        for (int c0 = 0; c0 < nsg; c0 += 64) {  // poll every chunk of 64 splits
          const int x = c0 + lane;
          uint32_t spins = 0;
          while (true) {
            bool ok = true;
            float2 v = make_float2(-INFINITY, 0.f);
            if (x < nsg) v = read_slot(x, ok);
            if (c0 == 0) v0 = v;
            if (__ballot(!ok) == 0ull) break;
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
              if (lane == 0) atomicOr(p.ws.err, kErrSpinTimeout);
              break;
            }
          }
        }
        auto slot_value = [&](int c0, int x) -> float2 {
          bool ok;
          return c0 == 0 ? v0 : (x < nsg ? read_slot(x, ok) : make_float2(-INFINITY, 0.f));
        };
        float Mloc = -INFINITY;
        for (int c0 = 0; c0 < nsg; c0 += 64) Mloc = fmaxf(Mloc, slot_value(c0, c0 + lane).x);
        const float M = wave_max(Mloc);
        uint64_t carry = 0;
        for (int c0 = 0; c0 < nsg; c0 += 64) {
          const int x = c0 + lane;
          const float2 v = slot_value(c0, x);
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
          // candidate points of this split: systematic and stratified points
          // are ordered by k, so only a short range of k can fall in this
          // split's probability range (one extra point on each side is
          // tested exactly below); i.i.d. points are all tested
          const double Z = (double)carry;
          sh.Z[g] = Z;
          const double lo = sh.Olo[g] / Z * (double)S, hi = sh.Ohi[g] / Z * (double)S;
          int klo = 0, khi = S - 1;
          if (p.mode == 2) {
            klo = max(0, (int)ceil(lo - sh.usys[g]) - 1);
            if (!is_last) khi = min(S - 1, (int)ceil(hi - sh.usys[g]) + 1);
          } else if (p.mode == 1) {
            klo = max(0, (int)floor(lo) - 1);
            if (!is_last) khi = min(S - 1, (int)ceil(hi) + 1);
          }
          sh.klo[g] = klo;
          sh.ncand[g] = max(0, khi - klo + 1);
        }
      }
      __syncthreads();

      // ---- stratum points in this split's range, CDF search -------------------
      // one candidate point per thread; the per-head constants are read once
      // into registers and selected with compare chains (no LDS round trips)
      {
        double Zh[G], Ol[G], Oh[G], Rs[G], Us[G];
        int Kl[G], first[G + 1];
        first[0] = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          Zh[g] = sh.Z[g];
          Ol[g] = sh.Olo[g];
          Oh[g] = sh.Ohi[g];
          Rs[g] = sh.rs[g];
          Us[g] = sh.usys[g];
          Kl[g] = sh.klo[g];
          first[g + 1] = first[g] + sh.ncand[g];
        }
        for (int pi = tid; pi < first[G]; pi += kThreads) {
          int g = 0;
#pragma unroll
          for (int x = 1; x < G; ++x) g = pi >= first[x] ? x : g;
          double Z = Zh[0], O = Ol[0], Ohg = Oh[0], r = Rs[0], u = Us[0];
          int k = pi - first[0] + Kl[0];
#pragma unroll
          for (int x = 1; x < G; ++x) {
            if (g == x) {
              Z = Zh[x];
              O = Ol[x];
              Ohg = Oh[x];
              r = Rs[x];
              u = Us[x];
              k = pi - first[x] + Kl[x];
            }
          }
          const uint32_t* ug = uni + g * kMaxS;
          double t;
          if (p.mode == 2) t = ((double)k + u) / (double)S;
          else if (p.mode == 1) t = ((double)k + (double)ug[k] * 0x1.0p-24) / (double)S;
          else t = (double)ug[k] * 0x1.0p-24;
          const double tz = t * Z;
          if (tz < O || (!is_last && tz >= Ohg)) continue;
          const int j = key_of(cdf + g * kPad, len, (float)((tz - O) / r));
          atomicAdd(&cnt[g * kSplit + j], 1u);
          atomicAdd(&sh.npts[g], 1);
          atomicOr(&sh.bits[j >> 5], 1u << (j & 31));
          if (p.idx_out) {
            int pos = k;
            if (p.mode == 0) {  // rank among the S uniforms, ties by stream index
              pos = 0;
              for (int x = 0; x < S; ++x) pos += (ug[x] < ug[k]) || (ug[x] == ug[k] && x < k);
            }
            p.idx_out[(size_t)(b * p.Hq + h0 + g) * S + pos] = k0 + j;
          }
        }
      }
      __syncthreads();

      // ---- distinct selected keys, in key order (one wave) -------------------
      if (w == 0) {
        uint32_t v = (sh.bits[lane >> 1] >> ((lane & 1) * 16)) & 0xFFFFu;  // keys 16*lane .. +15
        const int nb = __popc(v);
        const int incl = wave_incl_scan_dpp(nb);
        int pos = incl - nb;
        while (v) {
          const int bit = __ffs(v) - 1;
          v &= v - 1;
          list[pos++] = (uint32_t)(lane * 16 + bit);
        }
        if (lane == 63) sh.n_distinct = incl;
      }
      __syncthreads();

      // ---- gather-add: each distinct row once, added `count` times ---------
      // A row is spread over LPR lanes (8 features each) and replicated for
      // GH heads, so a lane accumulates its own head(s) over the rows of its
      // wave and no cross-lane sum is needed unless a wave holds RG > 1 rows.
      {
        constexpr int LPR = D / 8;
        constexpr int GH = (G * LPR <= 64) ? G : 64 / LPR;  // heads per row copy
        constexpr int HPL = G / GH;                          // heads per lane
        constexpr int RG = 64 / (LPR * GH);                  // rows per wave instruction
        constexpr int UNR = 4;                               // rows in flight per lane
        const int rg = lane / (LPR * GH), gh = (lane / LPR) % GH, c = lane % LPR;
        const _Float16* Vb = (const _Float16*)p.V + ((size_t)(b * p.Hkv + hk) * p.max_n_k + k0) * D;
        float acc[HPL][8];
#pragma unroll
        for (int x = 0; x < HPL; ++x)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[x][e] = 0.f;
        const int nd = sh.n_distinct;
        for (int i0 = 0; i0 < nd; i0 += kWaves * RG * UNR) {
          uint4 vv[UNR];
          int jj[UNR];
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            const int i = i0 + (u * kWaves + w) * RG + rg;
            jj[u] = i < nd ? (int)list[i] : -1;
            vv[u] = *(const uint4*)(Vb + (size_t)max(jj[u], 0) * D + c * 8);  // key 0 of the split when idle
          }
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            if (jj[u] < 0) continue;
            float f[8];
            unpack8(vv[u], f);
#pragma unroll
            for (int x = 0; x < HPL; ++x) {
              const float cf = (float)cnt[(gh + GH * x) * kSplit + jj[u]];  // count * v is exact
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[x][e] = fmaf(cf, f[e], acc[x][e]);
            }
          }
        }
        if constexpr (RG > 1) {
#pragma unroll
          for (int x = 0; x < HPL; ++x)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              for (int m = LPR * GH; m < 64; m <<= 1) acc[x][e] += __shfl_xor(acc[x][e], m, 64);
        }
        __syncthreads();  // `list` aliases `red`
        if (rg == 0) {
#pragma unroll
          for (int x = 0; x < HPL; ++x)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[w * G * D + (gh + GH * x) * D + c * 8 + e] = acc[x][e];
        }
      }
      __syncthreads();
      // ---- add this split's share into the output rows ----------------------
      for (int i = tid; i < G * D; i += kThreads) {
        if (sh.npts[i / D] == 0) continue;  // no point of this head fell here
        float v = red[i];
#pragma unroll
        for (int x = 1; x < kWaves; ++x) v += red[x * G * D + i];
        atomic_add_dev(p.out + (size_t)(b * p.Hq + h0) * D + i, v / (float)S);
      }
      if (tid == 0 && entered == 0xffffffffu) entered = atomic_add_dev(p.ws.exits, 1u);
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
  // ---- the last workgroup to exit advances the launch number ---------------
  if (tid == 0 && entered == 0xffffffffu) {  // a workgroup that published nothing
    wait_memory();                            // its read of the launch number is complete
    entered = atomic_add_dev(p.ws.exits, 1u);
  }
  if (tid == 0 && entered == (uint32_t)(p.grid - 1)) {
    store_dev(p.ws.exits, 0u);
    store_dev(p.ws.epoch, launch_tag());
  }
}

template <int D, int G>
size_t lds_bytes() { return Lds<D, G>::bytes; }

template <int D, int G, bool BERN, int OCC>
int capacity_t() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  auto fn = decode_kernel<D, G, BERN, OCC>;
  const size_t lds = lds_bytes<D, G>();
  (void)hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess) return 0;
  return per_cu * cus;
}

template <int D, int G, bool BERN, int OCC>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const size_t lds = lds_bytes<D, G>();
  hipLaunchKernelGGL((decode_kernel<D, G, BERN, OCC>), dim3(p.grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <bool BERN, int OCC>
hipError_t dispatch(const DecodeParams& p, hipStream_t stream) {
#define SANTA_CASE(DD, GG) \
  if (p.D == DD && p.G == GG) return launch_t<DD, GG, BERN, OCC>(p, stream);
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return hipErrorInvalidValue;
}

template <bool BERN, int OCC>
int capacity(int D, int G) {
#define SANTA_CASE(DD, GG) \
  if (D == DD && G == GG) return capacity_t<DD, GG, BERN, OCC>();
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return 0;
}

}  // namespace

int decode_capacity(int D, int G, bool bernoulli, int occ) {
  if (occ == 2) return bernoulli ? capacity<true, 2>(D, G) : capacity<false, 2>(D, G);
  return bernoulli ? capacity<true, 1>(D, G) : capacity<false, 1>(D, G);
}

hipError_t launch_decode(const DecodeParams& p, bool bernoulli, hipStream_t stream) {
  if (p.occ == 2) return bernoulli ? dispatch<true, 2>(p, stream) : dispatch<false, 2>(p, stream);
  return bernoulli ? dispatch<true, 1>(p, stream) : dispatch<false, 1>(p, stream);
}

}  // namespace santa
