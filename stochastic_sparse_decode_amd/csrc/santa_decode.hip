// SANTA stochastic sparse decode step: one fused, persistent kernel.
//
// Method: "Stochastic Sparse Attention for Memory-Bound Inference"
// (arXiv 2605.01910), abstract.  Every key is scored (the score stage still
// reads all of K); S key indices are drawn from the post-softmax distribution
// by inverse-CDF sampling (i.i.d., stratified, or systematic with a single
// offset), and only those value rows are gathered and added, divided by S,
// which estimates softmax(qK^T)V without bias.  In the Bernoulli qK^T mode
// the query is replaced by a stochastic ternary vector so that only the kept
// key features are read; a preparation kernel (bernoulli_prep, below) draws
// each group's query once per call.  (The Gumbel-max i.i.d. draws have their
// own kernels, santa_gumbel.hip.)
//
// Work decomposition (one GPU, gfx950):
//   work item = (sequence b, KV head, split of SPLIT keys).  Items of one KV
//   head ("group") are consecutive.  A workgroup (256 threads, 4 waves) takes
//   an item and streams that split's K rows once with 16-byte loads, scoring
//   the G query heads of the group from one read (GQA packing); the scores
//   stay in LDS.  After one barrier (the split maximum of each head), wave g
//   owns query head g for the rest of the item, with no further barriers:
//     1. fixed-point weights of its SPLIT keys (1024, or 512), SPLIT / 64
//        consecutive keys per lane, kept in registers with their exact sums;
//     2. publishes the split's (max, mass) as soon as the wave scan gives the
//        total, then polls the other splits' slots of the same head;
//     3. merges them: global max, exact integer split offsets, normaliser;
//     4. gets the number of sample points of each of its keys: for the
//        systematic and stratified schemes in closed form from the key's two
//        CDF edges, for i.i.d. draws by searching each point in the split's
//        CDF;
//     5. gathers each selected value row once, weighted by its count, and
//        adds the split's share of the estimate to the output row with fp32
//        device atomics (split 0 clears the row before it publishes), or, in
//        the deterministic mode, exactly in 64-bit integers that the group's
//        last split rounds once.
//
// Scheduling: `grid` workgroups are all resident (grid <= occupancy capacity).
// One item per workgroup when the items fit (VAR kOneItem: one workgroup per
// CU; kOneItemTwo: two per CU, with 512-key splits when 1024-key items would
// leave CUs idle); otherwise (kPersistent, two workgroups per CU) workgroup x
// takes the valid splits x, x + grid,
// x + 2 grid, ... and streams item k before it finishes item k - 1, so its
// wait for the other splits of item k - 1 overlaps its own K stream.  A wave
// only waits for splits of its own group, and every workgroup publishes its
// item of a round before it waits for any item of that round or a later
// one, so the waits always end as long as a group has no more splits than
// there are workgroups.  Every wait is bounded (kSpinLimit polls); a timeout
// sets an error bit instead of hanging.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "score_stage.h"

namespace santa {

namespace {

constexpr int kUniRow = kMaxS + 64;  // per-head row of uniforms

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Dynamic LDS of one workgroup:
//   sc  [nbuf][G][pad]   fp32 scores; then a head's weights (the i.i.d.
//                        scheme: its local CDF), then its list of selected
//                        keys (at most SPLIT entries + one spare slot per lane)
//   uni [G][kUniRow]     24-bit uniforms of the points (stratified, i.i.d.);
//                        finally the sums of the gather's row slots
//   cnt [G][SPLIT / 2]   i.i.d. points per key, two 16-bit counters a word
template <int D, int G, int NBUF, int SPLIT>
struct Lds {
  static constexpr int nbuf = NBUF;  // score buffers: the pipelined variant keeps two items
  static constexpr size_t sc_bytes = sizeof(float) * G * pad_of<SPLIT>();
  static constexpr size_t uni_bytes = sizeof(uint32_t) * G * kUniRow;
  static constexpr size_t cnt_bytes = sizeof(uint32_t) * G * (SPLIT / 2);
  static constexpr size_t bytes = nbuf * sc_bytes + uni_bytes + cnt_bytes;
};

// Launch variants of the sampling kernel.
enum Variant {
  kOneItem = 1,     // one work item per workgroup, one workgroup per CU
  kPersistent = 2,  // two workgroups per CU take the valid splits in turn
  kOneItemTwo = 3,  // one work item per workgroup, two workgroups per CU
};

struct Shared {
  float wmax[2][kWaves * 4][8];  // per score buffer: split maximum of each head, per wave and row of 16 lanes
  uint32_t epoch;  // launch tag of this launch
  // Bernoulli mode
  float A[8];
  uint64_t l1w[kWaves][8];  // budget variant: per-wave sums of |q| * 2^24
  float amax[kWaves][8];    // ternary queries: per-wave max |q|
  int wcount[kWaves];
  int nu;
};

// ---------------------------------------------------------------------------
// Score stage, Bernoulli qK^T: the ternary query keeps feature i of head g
// when u_i * A_g < |q_gi| (A_g = max_i |q_gi|, u_i shared by the group), with
// value sign(q_gi) * A_g.  K is stored as 64-key feature-major tiles, so each
// kept feature of a tile is one contiguous 128-byte row; only the union of
// the group's kept features is read, and each contributes by add/subtract.
// ---------------------------------------------------------------------------
// info[j] = (feature index << 16) | keep/sign bits of the j-th kept feature of
// the union; wt[j] = its fp16 query weight (+1, -1 or 0) for each head, and
// zero for every j past the union (so padded steps add nothing).  Head g's
// query is then A_g * wt (+ wt2 in the budget variant).
//
// Budget variant (BUDGET): feature i of head g is kept with probability
// pi = min(1, m |q_gi| / ||q_g||_1) and takes the value q_gi / pi: a clipped
// feature (pi = 1) keeps q_gi exactly (its fp16 value, in wt2), any other
// kept one sign(q_gi) ||q_g||_1 / m (a sign in wt, A_g = ||q_g||_1 / m).  With
// Q = |q| * 2^24 and U = the uniform's 24 bits (integers), keep <=>
// U * L1 < m * Q * 2^24 (L1 = sum of Q) and clipped <=> m * Q >= L1, both
// decided exactly in 128- and 64-bit integers.
template <int D, int G, bool BUDGET>
__device__ __forceinline__ void bernoulli_setup(const DecodeParams& p, int b, int hk, bool write_kept,
                                                Shared& sh, uint32_t* info, uint4* wt, uint4* wt2) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const _Float16* qb = (const _Float16*)p.q + (size_t)(b * p.Hq + hk * G) * D;
  constexpr int QW = (D + 63) / 64;  // waves that hold features
  // thread tid < D holds feature tid of every head and its uniform; the query
  // is read once, and its load overlaps the generator's arithmetic
  _Float16 qh[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qh[g] = tid < D ? qb[g * D + tid] : (_Float16)0;
  uint32_t ux = 0;
  if (tid < D) {
    const uint4 blk = stream_block(p.seed, (uint32_t)(b * p.Hkv + hk), kTagBernoulli, (uint32_t)(tid >> 2));
    ux = uniform_bits(word_of(blk, tid & 3));
  }
  // per wave: max |q_g| (ternary), or sum of |q_g| * 2^24 (budget; exact
  // integers, the sum below 2^47); every thread then combines the waves
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if constexpr (BUDGET) {
      uint64_t v = (uint64_t)((double)fabsf((float)qh[g]) * 16777216.0);
      for (int m = 1; m < 64; m <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
        v += ((uint64_t)hi << 32) | lo;
      }
      if (lane == 0 && w < QW) sh.l1w[w][g] = v;
    } else {
      float a = fabsf((float)qh[g]);
      for (int m = 1; m < 64; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
      if (lane == 0 && w < QW) sh.amax[w][g] = a;
    }
  }
  __syncthreads();
  float A[G];
  uint64_t L1[BUDGET ? G : 1];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if constexpr (BUDGET) {
      L1[g] = 0ull;
#pragma unroll
      for (int x = 0; x < QW; ++x) L1[g] += sh.l1w[x][g];
      A[g] = (float)((double)L1[g] * (1.0 / 16777216.0) / (double)p.budget);
    } else {
      A[g] = sh.amax[0][g];
#pragma unroll
      for (int x = 1; x < QW; ++x) A[g] = fmaxf(A[g], sh.amax[x][g]);
    }
  }
  if (tid < G) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (g == tid) sh.A[g] = A[g];
  }
  bool any = false;
  uint32_t bits = 0;
  uint32_t hw[4] = {0u, 0u, 0u, 0u};  // fp16 weights of the G heads, two per word
  uint32_t hq[4] = {0u, 0u, 0u, 0u};  // budget variant: exact query values of clipped features
  if (tid < D) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float qi = (float)qh[g];
      bool keep, clipped = false;
      if constexpr (BUDGET) {
        const uint64_t Q = (uint64_t)((double)fabsf(qi) * 16777216.0);
        const uint64_t mq = (uint64_t)p.budget * Q;  // below 2^47
        const uint64_t lhs_hi = __umul64hi((uint64_t)ux, L1[g]), lhs_lo = (uint64_t)ux * L1[g];
        const uint64_t rhs_hi = mq >> 40, rhs_lo = mq << 24;
        keep = lhs_hi < rhs_hi || (lhs_hi == rhs_hi && lhs_lo < rhs_lo);
        clipped = keep && mq >= L1[g];
      } else {
        // u * A < |q|  <=>  (x >> 8) * A < |q| * 2^24, exact in fp64
        keep = (double)ux * (double)A[g] < (double)fabsf(qi) * 16777216.0;
      }
      if (keep) bits |= (1u << (2 * g)) | ((qi < 0.f ? 1u : 0u) << (2 * g + 1));
      const uint32_t h16 = keep && !clipped ? (qi < 0.f ? 0xBC00u : 0x3C00u) : 0u;  // -1, +1 or 0 in fp16
      hw[g >> 1] |= h16 << (16 * (g & 1));
      if (clipped) hq[g >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, qh[g]) << (16 * (g & 1));
      any |= keep;
      if (write_kept) p.kept_out[(size_t)(b * p.Hq + hk * G + g) * D + tid] = keep ? 1 : 0;
    }
  }
  // compact the union of kept features in increasing feature order
  const uint64_t bal = __ballot(any);
  const int before = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0 && w < 2) sh.wcount[w] = __popcll(bal);
  __syncthreads();
  const int nu = (D > 64) ? sh.wcount[0] + sh.wcount[1] : sh.wcount[0];
  if (any) {
    const int pos = before + (w == 1 ? sh.wcount[0] : 0);
    info[pos] = ((uint32_t)tid << 16) | bits;
    wt[pos] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    if constexpr (BUDGET) wt2[pos] = make_uint4(hq[0], hq[1], hq[2], hq[3]);
  }
  for (int j = nu + tid; j < 128; j += kThreads) {
    wt[j] = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (BUDGET) wt2[j] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (tid == 0) sh.nu = nu;
  __syncthreads();
}

// The prepared query of a group (written by bernoulli_prep earlier in the
// same stream) into the workgroup's LDS: the union's size, the heads' scale
// factors, the kept-feature list and the heads' weights (the budget variant:
// and the clipped features' exact values).  Entry i of the record:
template <bool BUDGET>
__device__ __forceinline__ void bernoulli_put(int i, const uint4& v, Shared& sh, uint32_t* info, uint4* wt,
                                              uint4* wt2) {
  if (i == 0) {
    sh.nu = (int)v.x;
  } else if (i < 3) {
    sh.A[(i - 1) * 4 + 0] = __uint_as_float(v.x);
    sh.A[(i - 1) * 4 + 1] = __uint_as_float(v.y);
    sh.A[(i - 1) * 4 + 2] = __uint_as_float(v.z);
    sh.A[(i - 1) * 4 + 3] = __uint_as_float(v.w);
  } else if (i < 35) {
    info[(i - 3) * 4 + 0] = v.x;
    info[(i - 3) * 4 + 1] = v.y;
    info[(i - 3) * 4 + 2] = v.z;
    info[(i - 3) * 4 + 3] = v.w;
  } else if (i < 163) {
    wt[i - 35] = v;
  } else {
    if constexpr (BUDGET) wt2[i - 163] = v;
  }
}
template <bool BUDGET>
constexpr int bern_words() { return BUDGET ? kBernRecord : 163; }
template <bool BUDGET>
__device__ __forceinline__ void bernoulli_load(const DecodeParams& p, int group, Shared& sh, uint32_t* info,
                                               uint4* wt, uint4* wt2) {
  const uint4* rec = p.ws.bern + (size_t)group * kBernRecord;
  for (int i = threadIdx.x; i < bern_words<BUDGET>(); i += kThreads) bernoulli_put<BUDGET>(i, rec[i], sh, info, wt, wt2);
  __syncthreads();
}
// Draws every group's ternary (or budget) query once per call: one workgroup
// per (sequence, KV head) runs bernoulli_setup and stores its result as the
// group's record (and the kept-feature masks, when asked for, of every
// sequence); each work item of the decode kernel then loads its group's
// record instead of drawing the query again for every split.
template <int D, int G, bool BUDGET>
__global__ __launch_bounds__(kThreads) void bernoulli_prep(DecodeParams p) {
  __shared__ Shared sh;
  __shared__ uint32_t info[128];
  __shared__ uint4 wt[128];
  __shared__ uint4 wt2[BUDGET ? 128 : 1];
  const int group = blockIdx.x, b = group / p.Hkv, hk = group % p.Hkv;
  bernoulli_setup<D, G, BUDGET>(p, b, hk, p.kept_out != nullptr, sh, info, wt, wt2);  // ends with a barrier
  uint4* rec = p.ws.bern + (size_t)group * kBernRecord;
  constexpr int n = BUDGET ? kBernRecord : 163;
  auto a_of = [&](int g) -> uint32_t { return g < G ? __float_as_uint(sh.A[g]) : 0u; };
  for (int i = threadIdx.x; i < n; i += kThreads) {
    uint4 v;
    if (i == 0) {
      v = make_uint4((uint32_t)sh.nu, 0u, 0u, 0u);
    } else if (i < 3) {
      const int g0 = (i - 1) * 4;
      v = make_uint4(a_of(g0), a_of(g0 + 1), a_of(g0 + 2), a_of(g0 + 3));
    } else if (i < 35) {
      const int j = (i - 3) * 4;  // entries past the union are never read
      v = make_uint4(info[j], info[j + 1], info[j + 2], info[j + 3]);
    } else if (i < 163) {
      v = wt[i - 35];
    } else {
      v = BUDGET ? wt2[i - 163] : make_uint4(0u, 0u, 0u, 0u);
    }
    rec[i] = v;
  }
}

template <int D, int G, bool BUDGET>
__device__ __forceinline__ void score_bernoulli(const DecodeParams& p, int b, int hk, int k0, int len,
                                                float* cdf, float* mx, const Shared& sh, const uint32_t* info,
                                                const uint4* wt, const uint4* wt2) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int half = lane >> 5, t4 = (lane >> 3) & 3, ko = lane & 7;
  const int ti = w * 4 + t4;  // tile of this lane inside the split (16 tiles)
  const int tiles_per_head = p.max_n_k / kTile;
  constexpr int kPad = pad_of<kSplit>();  // the Bernoulli stage runs splits of kSplit keys
  // tiles past the sequence end re-read its last tile (results discarded)
  const int tile = min(k0 / kTile + ti, (k0 + len - 1) / kTile);
  const _Float16* tb = (const _Float16*)p.K + ((size_t)(b * p.Hkv + hk) * tiles_per_head + tile) * (size_t)(D * kTile);
  const int nu = sh.nu;
  float acc[G][8];                      // sums against the sign weights (factor A_g)
  float acc2[BUDGET ? G : 1][8];        // budget variant: against the clipped values (factor 1)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
#pragma unroll
  for (int g = 0; g < (BUDGET ? G : 1); ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc2[g][e] = 0.f;

  // A lane takes the kept features j = 2 x + half of the list, two steps at a
  // time: the two features' values of a key form one fp16 pair, and so do the
  // head's weights for them, so one v_dot2 (fp32 accumulate) adds both.
  constexpr int UNR = 8;  // steps (loads) per iteration, an even number
  const int steps = (nu + 1) / 2;
  for (int f0 = 0; f0 < steps; f0 += UNR) {
    uint4 kv[UNR];
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
      const int fi = 2 * (f0 + x) + half;
      const uint32_t e = info[fi < nu ? fi : 0];  // past the list: a kept row, weighted 0
      kv[x] = load_nt((const uint4*)(tb + (size_t)(e >> 16) * kTile + ko * 8));
    }
#pragma unroll
    for (int x = 0; x < UNR; x += 2) {
      const int j0 = 2 * (f0 + x) + half;  // j0 + 2 < 128: the table holds 128 entries
      const uint4 wa = wt[j0], wc = wt[j0 + 2];
      uint32_t wp[G], wq[BUDGET ? G : 1];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t a = word_of(wa, g >> 1), c = word_of(wc, g >> 1);
        wp[g] = __builtin_amdgcn_perm(c, a, (g & 1) ? 0x07060302u : 0x05040100u);
      }
      if constexpr (BUDGET) {
        const uint4 qa = wt2[j0], qc = wt2[j0 + 2];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t a = word_of(qa, g >> 1), c = word_of(qc, g >> 1);
          wq[g] = __builtin_amdgcn_perm(c, a, (g & 1) ? 0x07060302u : 0x05040100u);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t a = word_of(kv[x], i), c = word_of(kv[x + 1], i);
        const uint32_t klo = __builtin_amdgcn_perm(c, a, 0x05040100u);  // key 2i: (feature j0, j0 + 2)
        const uint32_t khi = __builtin_amdgcn_perm(c, a, 0x07060302u);  // key 2i + 1
#pragma unroll
        for (int g = 0; g < G; ++g) {
          acc[g][2 * i] = __builtin_amdgcn_fdot2(as_h2(wp[g]), as_h2(klo), acc[g][2 * i], false);
          acc[g][2 * i + 1] = __builtin_amdgcn_fdot2(as_h2(wp[g]), as_h2(khi), acc[g][2 * i + 1], false);
          if constexpr (BUDGET) {
            acc2[g][2 * i] = __builtin_amdgcn_fdot2(as_h2(wq[g]), as_h2(klo), acc2[g][2 * i], false);
            acc2[g][2 * i + 1] = __builtin_amdgcn_fdot2(as_h2(wq[g]), as_h2(khi), acc2[g][2 * i + 1], false);
          }
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
      float s = tot * sc;
      if constexpr (BUDGET) s = fmaf(acc2[g][e] + __shfl_xor(acc2[g][e], 32, 64), p.scale, s);
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
// weight: w = exp(s - m) in (0, 1] becomes q = trunc(w * 2^31), and the local
// CDF c_j = q_0 + ... + q_j is an exact integer (held in doubles, whose sums
// of such integers are exact and so independent of the order of additions).
// The split masses merged across the group are integers too, so the split
// offsets O_s are exact, nondecreasing and identical in every workgroup.  In
// global units the right edge of key j of split s is
//   X_j = min(O_s + r_s c_j, O_{s+1}),  r_s = exp(m_s - M),
// and the last key of a split ends exactly at O_{s+1}, so the keys of all
// splits tile [0, Z) without gaps or overlaps.  A point t selects the key
// whose interval [X_{j-1}, X_j) holds t Z (the inverse CDF, half-open).
// ---------------------------------------------------------------------------
constexpr float kFix = 2147483648.0f;  // 2^31
constexpr int kPollSleep = 4;          // s_sleep argument between poll rounds (64 clocks each)

// e^x for x <= 0 (x finite, or a large negative stand-in for a masked key),
// within about 2 ulp: the hardware base-2 exponential of t = fl(x log2 e),
// corrected to first order by the rounding residual of that product (the
// residual is below half an ulp of t, so the dropped second-order term is far
// below fp32 resolution).  Branch-free, 8 instructions.
__device__ __forceinline__ float exp_nonpos(float x) {
  constexpr float kLog2e = 1.44269502162933349609375f;  // log2(e) rounded to fp32
  constexpr float kLog2eLo = 1.925963033500011e-08f;    // log2(e) - kLog2e
  constexpr float kLn2 = 0.693147180559945309f;
  const float t = x * kLog2e;
  const float r = fmaf(x, kLog2e, -t) + x * kLog2eLo;   // x log2(e) - t
  const float p = __builtin_amdgcn_exp2f(t);
  return fmaf(p, r * kLn2, p);
}

// Orders this wave's LDS accesses: a wave's LDS operations complete in
// program order, so after this point every lane reads what any lane of the
// same wave wrote before it (the fence keeps the compiler from moving LDS
// accesses across it).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t u, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over segments of SEG lanes (SEG = 8 or 16; i = lane
// index in its segment) of doubles that hold integers below 2^53, so every
// partial sum is exact: DPP row shifts by 1, 2, 4 (and 8), a lane taking
// nothing from across its segment's start.
template <int SEG>
__device__ __forceinline__ double seg_scan_exact(double c, int i) {
  static_assert(SEG == 8 || SEG == 16, "segment width");
  auto step = [&](auto ctrl, int k) {
    const double sh = __builtin_bit_cast(double, dpp_u64<decltype(ctrl)::value, 0xF>(__builtin_bit_cast(uint64_t, c)));
    c += (SEG == 16 || i >= k) ? sh : 0.0;
  };
  step(std::integral_constant<int, 0x111>{}, 1);
  step(std::integral_constant<int, 0x112>{}, 2);
  step(std::integral_constant<int, 0x114>{}, 4);
  if constexpr (SEG == 16) step(std::integral_constant<int, 0x118>{}, 8);
  return c;
}

// Number of keys j < len with c_j <= tau (c nondecreasing): the first key
// whose CDF value exceeds tau, clamped to len - 1.  Branch-free radix-4
// search over the split's SPLIT slots: each level reads three probes together
// and keeps the quarter they select (the probe test is true, then false, along
// the split), so five dependent rounds of LDS reads instead of ten for 1024
// slots; for 512 slots one binary level comes first.  Probes stay below
// SPLIT - 1.
template <int SPLIT>
__device__ __forceinline__ int key_of(const float* c, int len, float tau) {
  static_assert(SPLIT == 1024 || SPLIT == 512, "radix-4 levels (and one binary level) cover the split");
  int lo = 0;
  if constexpr (SPLIT == 512) {
    const int p1 = 255;
    lo += (p1 < len && c[lidx(p1)] <= tau) ? 256 : 0;
  }
#pragma unroll
  for (int step = (SPLIT == 512 ? 64 : SPLIT / 4); step >= 1; step >>= 2) {
    const int p1 = lo + step - 1, p2 = lo + 2 * step - 1, p3 = lo + 3 * step - 1;
    const float v1 = c[lidx(p1)], v2 = c[lidx(p2)], v3 = c[lidx(p3)];
    const int adv = (p1 < len && v1 <= tau ? 1 : 0) + (p2 < len && v2 <= tau ? 1 : 0) +
                    (p3 < len && v3 <= tau ? 1 : 0);
    lo += adv * step;
  }
  return lo < len ? lo : len - 1;
}

// ---------------------------------------------------------------------------
// The fused kernel.
// ---------------------------------------------------------------------------
// VAR (Variant):
//  kOneItem, kOneItemTwo: every work item has its own workgroup (grid =
//  total_items, launched only then; one or two workgroups per CU): stream the
//  split, publish, wait, finish; no item loop.
//  kPersistent: two workgroups per CU take the valid splits round-robin and
//  pipeline them: stream item k and publish its statistics, then finish item
//  k - 1 (whose group has normally published everything by then), so the
//  sampling tail of one item never stalls the K stream of the next.
// SPLIT: keys per work item, 1024, or 512 for the plain fp16 cache when the
// problem has too few 1024-key splits to give every CU two.
template <int D, int G, int KIND, int VAR, int SPLIT>
__global__ __launch_bounds__(kThreads, VAR == kOneItem ? 1 : 2) void decode_kernel(DecodeParams p) {
  constexpr bool BUDGET = KIND == kKeyBernoulliBudget;
  constexpr bool BERN = KIND == kKeyBernoulli || BUDGET;
  constexpr bool PAGED = KIND == kKeyF16Paged;
  constexpr int OCC = VAR == kOneItem ? 1 : 2;  // workgroups per CU
  constexpr bool LOOP = VAR == kPersistent;
  constexpr int kPer = SPLIT / 64;           // keys per lane in the per-head steps
  constexpr int kPad = pad_of<SPLIT>();
  static_assert(SPLIT == kSplit || KIND == kKeyF16, "shorter splits are built for the plain fp16 cache only");
  extern __shared__ __align__(16) unsigned char smem[];
  using L = Lds<D, G, LOOP ? 2 : 1, SPLIT>;
  uint32_t* uni = (uint32_t*)(smem + L::nbuf * L::sc_bytes);                  // [G][kUniRow]
  uint32_t* cntw = (uint32_t*)(smem + L::nbuf * L::sc_bytes + L::uni_bytes);  // [G][SPLIT / 2]
  auto score_buf = [&](int i) -> float* { return (float*)(smem + (size_t)i * L::sc_bytes); };  // [G][kPad]
  __shared__ Shared sh;
  __shared__ uint32_t binfo[BERN ? 128 : 1];  // Bernoulli kept-feature union
  __shared__ uint4 bwt[BERN ? 128 : 1];       // and its per-head fp16 weights
  __shared__ uint4 bwt2[BUDGET ? 128 : 1];    // budget variant: exact values of clipped features
  // paged cache: the block of each block-sized key range of the item in
  // score buffer wb (validated; an out-of-range entry reads block 0)
  __shared__ int pblk[PAGED ? 2 : 1][PAGED ? SPLIT / 16 : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int S = p.S;
  // Launch tag of the statistics slots.  The launch count is the sum of the
  // workspace's kLaunchCounters 64-bit counters (one per 128-byte line, so that
  // the adds of a launch do not all queue on one address), and every launch
  // adds exactly kLaunchUnit to that sum: workgroup 0 adds kLaunchUnit -
  // (grid - 1) to counter 0, every other workgroup x adds 1 to counter
  // x mod kLaunchCounters, each only after its own reads of all the counters
  // have completed.  The counters only grow, so a sum read during launch L,
  // even from values read one at a time, is at least L kLaunchUnit and lacks
  // at least the reader's own add: it lies in [L kLaunchUnit, (L + 1)
  // kLaunchUnit).  All workgroups of a launch derive the same launch number,
  // and a slot left by an earlier launch (or an earlier replay of a captured
  // graph) never carries this launch's tag.  No workgroup waits for the add.
  uint64_t lc = 0ull;  // lane i < kLaunchCounters of wave 0: counter i as read (issued with the first item)
  bool tagged = false;  // the launch tag is in sh.epoch
  // One field of each 64-byte line of the arguments is fetched here, so all
  // lines arrive in one scalar round trip instead of one after another where
  // their fields are first used (the first K load waits for them).
  {
    const void* k_ptr = p.K;
    const int32_t* nk_ptr = p.n_k;
    const void* v_ptr = p.V;
    const uint32_t* err_ptr = p.ws.err;
    const void* q_ptr = p.q;
    const uint64_t* lc_ptr = p.ws.launches;
    const float* ks_ptr = p.k_scale;
    const int ns_ = p.ns, mnk = p.max_n_k, hkv = p.Hkv, items = p.total_items;
    asm volatile("" ::"s"(k_ptr), "s"(nk_ptr), "s"(q_ptr), "s"(v_ptr), "s"(err_ptr), "s"(lc_ptr), "s"(ks_ptr), "s"(ns_),
                 "s"(mnk), "s"(hkv), "s"(items));
  }
  auto tag_of = [](uint64_t c) -> uint32_t {
    const uint32_t t = (uint32_t)(c / kLaunchUnit) + 1u;
    return t == 0u ? 1u : t;
  };
  const uint64_t my_add = blockIdx.x == 0 ? kLaunchUnit - (uint64_t)(p.grid - 1) : 1ull;
  bool counted = false;  // thread 0: this workgroup's add has been issued

  // ---- one work item: (sequence b, KV head hk, split s) ---------------------
  struct ItemCtx {
    int group, s, b, hk, h0, nsg, k0, len;
    bool valid, active, is_last;
  };
  // The item's fields.  `first_rows` runs between the read of the sequence
  // length and its first use: loads it issues are younger than the length's,
  // so waiting for the length does not wait for them.
  auto describe = [&](int item, auto&& first_rows) -> ItemCtx {
    ItemCtx it;
    it.group = item / p.ns;
    it.s = item % p.ns;
    it.b = it.group / p.Hkv;
    it.hk = it.group % p.Hkv;
    it.h0 = it.hk * G;
    // a scalar read (the lengths do not change during the kernel): waiting for
    // it does not wait for vector loads issued after it
    const int n = *(const __attribute__((address_space(4))) int32_t*)(p.n_k + it.b);
    // the counter read is issued after the length read, so waiting for the
    // length does not wait for it; it is first needed after the score stage
    if (tid < kLaunchCounters && !tagged) lc = load_dev(p.ws.launches + tid * kLaunchStride);
    it.k0 = it.s * SPLIT;
    first_rows(it);
    it.valid = n >= 1 && n <= p.max_n_k;
    it.nsg = it.valid ? (n + SPLIT - 1) / SPLIT : 0;
    it.active = it.valid && it.s < it.nsg;
    it.len = it.active ? min(SPLIT, n - it.k0) : 0;
    it.is_last = it.s == it.nsg - 1;
    return it;
  };

  // start of key (or value) row j of an item's split, for the KV head's
  // contiguous block or through the block table
  auto row_of = [&](const void* base, const ItemCtx& it, int wb, int j) -> const _Float16* {
    if constexpr (PAGED) {
      const int blk = pblk[wb][j >> p.lg_block];
      const size_t slab = ((size_t)blk * p.Hkv + it.hk) << p.lg_block;  // first row of the (block, head) slab
      return (const _Float16*)base + (slab + (size_t)(j & ((1 << p.lg_block) - 1))) * D;
    } else {
      return (const _Float16*)base + ((size_t)(it.b * p.Hkv + it.hk) * p.max_n_k + it.k0 + j) * D;
    }
  };

  // ---- per query head (wave g owns head g) ---------------------------------
  // Fixed-point weights q of the keys lane*kPer .. lane*kPer+kPer-1 of head
  // g, the lane's exclusive prefix and the split total (integers below 2^53
  // held in doubles, so every partial sum is exact in any order).
  struct Weights {
    uint32_t q[kPer];
    double excl, lsum, total;  // the lane's exclusive prefix and own sum, the split's total
    float m;
  };
  auto weights = [&](const ItemCtx& it, int g, const float* scb, int wb, Weights& wt) {
        const int len = it.len;
        const float* cg = scb + g * kPad;
        // one value per wave (Bernoulli stage) or per wave and row of 16 lanes
        constexpr int kParts = BERN ? kWaves : kWaves * 4;
        float m = sh.wmax[wb][0][g];
#pragma unroll
        for (int x = 1; x < kParts; ++x) m = fmaxf(m, sh.wmax[wb][x][g]);

        uint64_t acc = 0;  // at most kPer * 2^31
        {
          float sv[kPer];
#pragma unroll
          for (int i = 0; i < kPer; ++i) sv[i] = cg[lidx(lane * kPer + i)];
          if (len == SPLIT) {
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
              const uint32_t q = (uint32_t)(exp_nonpos(sv[i] - m) * kFix);  // trunc(w * 2^31), exact: w <= 1
              acc += q;
              wt.q[i] = q;
            }
          } else {
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
              // rows past the split's end hold unrelated LDS contents: their
              // argument is replaced by -1000, whose exponential is 0 in fp32
              const float wv = exp_nonpos(lane * kPer + i < len ? sv[i] - m : -1000.f);
              const uint32_t q = (uint32_t)(wv * kFix);
              acc += q;
              wt.q[i] = q;
            }
          }
        }
        const double incl = wave_incl_scan_exact((double)acc);
        wt.lsum = (double)acc;
        wt.excl = incl - wt.lsum;  // exact: all values are integers below 2^53
        wt.total = readlane_f64(incl, 63);
        wt.m = m;
  };

  // The pipelined variant finishes an item after streaming the next one: the
  // weights stay in the item's score buffer (each score of head g replaced by
  // its weight) instead of being computed a second time.  Only wave g
  // accesses head g's row from here on, and one wave's LDS accesses complete
  // in order.
  auto stash_weights = [&](int g, float* scb, const Weights& wt) {
    uint32_t* cg = (uint32_t*)(scb + g * kPad);
#pragma unroll
    for (int i = 0; i < kPer; ++i) cg[lidx(lane * kPer + i)] = wt.q[i];
  };
  auto reload_weights = [&](int g, const float* scb, Weights& wt) {
    const uint32_t* cg = (const uint32_t*)(scb + g * kPad);
    uint64_t acc = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      wt.q[i] = cg[lidx(lane * kPer + i)];
      acc += wt.q[i];
    }
    const double incl = wave_incl_scan_exact((double)acc);
    wt.lsum = (double)acc;
    wt.excl = incl - wt.lsum;
    wt.total = readlane_f64(incl, 63);
  };

  // Statistics slots of head g of an item's group: [group][head][split], each
  // slot (tag:32 | max bits, tag:32 | mass bits) at the start of p.slot_words
  // 8-byte words.
  auto slot_row = [&](const uint64_t* base, const ItemCtx& it, int g) -> const uint64_t* {
    return base + ((size_t)it.group * G + g) * p.ns * p.slot_words;
  };
  // Publish head g's (split max, split mass).
  auto publish = [&](const ItemCtx& it, int g, const Weights& wt) {
        const uint32_t tag = sh.epoch;
        // Each half of the 16-byte slot carries the launch tag, so a reader
        // accepts it only when both halves were written by this launch.  Split
        // 0 cleared the output rows (the exact rows in the deterministic mode)
        // before its score stage; the wait makes sure those stores have
        // completed (they have, long ago) before any split can see its slot
        // and add.
        if (it.s == 0) wait_memory();
        if (lane < 2) {
          const uint64_t t = (uint64_t)tag << 32;
          uint64_t* sl = const_cast<uint64_t*>(slot_row(p.ws.stats, it, g)) + it.s * p.slot_words + lane;
          store_dev(sl, t | __float_as_uint(lane == 0 ? wt.m : (float)wt.total));
        }
        // this workgroup's share of the launch counter (its read has completed:
        // the value is in LDS); issued after the publish so that no wait before
        // a publish covers its round trip
        if (tid == 0 && !counted) {
          atomic_add_noret(p.ws.launches + (blockIdx.x % kLaunchCounters) * kLaunchStride, my_add);
          counted = true;
        }
  };

  // The sampling tail of head g in two halves: tail_a waits for the group's
  // statistics, places the points and issues the first value loads; tail_b
  // adds the value rows into the output.
  constexpr int kVU = 4;  // value loads per lane per round of the gather
  constexpr int LPR = D / 8, RPW = 64 / LPR;
  static_assert(2 * RPW * D <= kUniRow && D % 64 == 0, "exact row-slot sums fit the head's uniform row");
  struct Gather {
    int nsel;
    uint32_t ee[kVU];
    uint4 vv[kVU];
  };
  // One round of reads of head g's statistics slots: the first kRegChunks * 64
  // splits, one 16-byte read per slot (both halves, each carrying the launch
  // tag), issued together so that a round is one round trip, and kept in
  // registers.  A lane whose slot already carries this launch's tag, or lies
  // past the group's last split, reads nothing: the waiting waves request
  // only the slots still missing, so the polls load the memory system less
  // while the last splits finish.
  constexpr int kRegChunks = 4;
  struct Poll {
    u32x4 sl[kRegChunks];  // (m bits, tag, mass bits, tag)
    bool seen[kRegChunks];
  };
  // Chunks past the group's last split are not read.
  auto poll_issue = [&](const ItemCtx& it, int g, Poll& pl) {
    const uint64_t* slots = slot_row(p.ws.stats, it, g);
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
      if (c > 0 && c * 64 >= it.nsg) break;
      if (!pl.seen[c]) pl.sl[c] = load_dev16(slots + (c * 64 + lane) * p.slot_words);
    }
  };
  auto tail_a = [&](const ItemCtx& it, int g, float* scb, int wb, const Weights& wt, Gather& gt, bool stashed) {
        const int s = it.s, len = it.len, k0 = it.k0, nsg = it.nsg, b = it.b, hk = it.hk, h0 = it.h0;
        const bool is_last = it.is_last;
        const uint32_t tag = sh.epoch;
        const uint64_t* slots = slot_row(p.ws.stats, it, g);
        const uint32_t row = (uint32_t)(b * p.Hq + h0 + g);
        float* cg = scb + g * kPad;
        // while the other splits finish: the points' uniforms, and for i.i.d.
        // draws the fp32 local CDF to search and cleared counters
        uint32_t* ug = uni + g * kUniRow;
        uint32_t* cw = cntw + g * (SPLIT / 2);
        if (p.mode != 2) {
          const uint32_t stag = p.mode == 1 ? kTagStratified : kTagIid;
          const int nb = (S + 3) >> 2;
          for (int kb = lane; kb < nb; kb += 64) {
            const uint4 blk = stream_block(p.seed, row, stag, (uint32_t)kb);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kb * 4 + e < S) ug[kb * 4 + e] = uniform_bits(word_of(blk, e));
          }
        }
        if (p.mode == 0) {
          double cum = wt.excl;
#pragma unroll
          for (int i = 0; i < kPer; ++i) {
            cum += (double)wt.q[i];
            if (lane * kPer + i < len) cg[lidx(lane * kPer + i)] = (float)cum;  // nondecreasing
          }
          for (int i = lane; i < SPLIT / 2; i += 64) cw[i] = 0u;
        } else if (!stashed) {
          stash_weights(g, scb, wt);  // read back by the lanes that place points
        }
        const double usys = p.mode == 2 ? uniform_f64(stream_block(p.seed, row, kTagSystematic, 0u).x) : 0.0;
        wave_lds_sync();

        // 3. wait for every split of the group, merge
        double Z = 0.0, Olo = 0.0, Ohi = 0.0, rs = 0.0;
        {
          // The slots of the first kRegChunks * 64 splits are read together
          // and kept in registers (one round trip however many splits there
          // are up to that bound); splits beyond it are polled and re-read a
          // chunk of 64 at a time.
          auto read_slot = [&](int x, bool& ok) -> float2 {
            const u32x4 a = load_dev16(slots + x * p.slot_words);
            ok = a.y == tag && a.w == tag;
            return make_float2(__uint_as_float(a.x), __uint_as_float(a.z));
          };
          float2 v[kRegChunks];
          {
            Poll pl;
#pragma unroll
            for (int c = 0; c < kRegChunks; ++c) {
              pl.seen[c] = c * 64 + lane >= nsg;
              pl.sl[c] = u32x4{0u, 0u, 0u, 0u};
            }
            auto test = [&]() -> bool {
              bool all = true;
#pragma unroll
              for (int c = 0; c < kRegChunks; ++c) {
                if (c > 0 && c * 64 >= nsg) break;
                pl.seen[c] = pl.seen[c] || (pl.sl[c].y == tag && pl.sl[c].w == tag);
                all = all && pl.seen[c];
              }
              return __ballot(!all) == 0ull;
            };
            poll_issue(it, g, pl);
            if (!test()) {
              uint32_t spins = 0;
              while (true) {
                __builtin_amdgcn_s_sleep(kPollSleep);
                if (++spins > kSpinLimit) {
                  if (lane == 0) atomicOr(p.ws.err, kErrSpinTimeout);
                  break;
                }
                poll_issue(it, g, pl);
                if (test()) break;
              }
            }
#pragma unroll
            for (int c = 0; c < kRegChunks; ++c)
              v[c] = c * 64 + lane < nsg ? make_float2(__uint_as_float(pl.sl[c].x), __uint_as_float(pl.sl[c].z))
                                         : make_float2(-INFINITY, 0.f);
          }
          // Beyond the register chunks: a lane stops reading once its slot
          // carries this launch's tag, and the wave sleeps between rounds, so
          // waiting waves add little traffic to the memory channels that the
          // splits still streaming K are using.
          for (int c0 = kRegChunks * 64; c0 < nsg; c0 += 64) {
            const int x = c0 + lane;
            bool ok = x >= nsg;
            uint32_t spins = 0;
            while (true) {
              if (!ok) (void)read_slot(x, ok);
              if (__ballot(!ok) == 0ull) break;
              __builtin_amdgcn_s_sleep(kPollSleep);
              if (++spins > kSpinLimit) {
                if (lane == 0) atomicOr(p.ws.err, kErrSpinTimeout);
                break;
              }
            }
          }
          auto far_slot = [&](int x) -> float2 {
            bool ok;
            return x < nsg ? read_slot(x, ok) : make_float2(-INFINITY, 0.f);
          };
          float Mloc = -INFINITY;
#pragma unroll
          for (int c = 0; c < kRegChunks; ++c) Mloc = fmaxf(Mloc, v[c].x);
          for (int c0 = kRegChunks * 64; c0 < nsg; c0 += 64) Mloc = fmaxf(Mloc, far_slot(c0 + lane).x);
          const float M = wave_max(Mloc);
          // Split masses in the units of M: Q_s = trunc(mass_s r_s), an integer
          // (the product of two fp32 values is exact in fp64), below 2^41 each
          // and 2^49 in total, so the double scan is exact.
          double carry = 0.0;
          auto merge_chunk = [&](int c0, float2 sv) {
            const int x = c0 + lane;
            const float r = x < nsg ? exp_nonpos(sv.x - M) : 0.f;
            const double Q = x < nsg ? trunc((double)sv.y * (double)r) : 0.0;
            const double inc = wave_incl_scan_exact(Q) + carry;
            if (s >= c0 && s < c0 + 64) {
              Olo = readlane_f64(inc - Q, s - c0);
              Ohi = readlane_f64(inc, s - c0);
              rs = (double)__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r), s - c0));
            }
            carry = readlane_f64(inc, 63);
          };
#pragma unroll
          for (int c = 0; c < kRegChunks; ++c)
            if (c * 64 < nsg) merge_chunk(c * 64, v[c]);
          for (int c0 = kRegChunks * 64; c0 < nsg; c0 += 64) merge_chunk(c0, far_slot(c0 + lane));
          Z = carry;
        }

        // 4. points per key and the list of selected keys (key | count << 16),
        // in key order, in the head's score row (free by now: the i.i.d.
        // search is done with it, the other schemes read the weights there
        // only at keys above any list position written so far); the sampled
        // indices (optional output), ascending
        uint32_t* list = (uint32_t*)cg;
        int* ix = p.idx_out ? p.idx_out + (size_t)row * S : nullptr;
        int nsel = 0;
        if (p.mode == 0) {
          // i.i.d.: the points in [Olo, Ohi) (the last split: [Olo, Z)) are
          // searched; earlier points are counted for the numbering.  The
          // in-range points are first packed to the front of the head's
          // uniform row (in place: every pass reads its 64 entries before any
          // lane writes, and writes only below the next pass's entries), so
          // the wave runs one search per 64 in-range points rather than one
          // per 64 points of the head.
          int cnt[kPer];
          int before = 0;
          int nin = 0;
          float* tin = (float*)ug;
          for (int k0p = 0; k0p < S; k0p += 64) {
            const int k = k0p + lane;
            bool in = false;
            float x = 0.f;
            if (k < S) {
              const double tz = (double)ug[k] * 0x1.0p-24 * Z;
              if (tz < Olo) {
                ++before;
              } else if (is_last || tz < Ohi) {
                in = true;
                x = (float)((tz - Olo) / rs);
              }
            }
            const uint64_t inm = __ballot(in);
            wave_lds_sync();  // the pass's reads are done before its writes
            if (in) tin[nin + __popcll(inm & ((1ull << lane) - 1ull))] = x;
            nin += __popcll(inm);
          }
          wave_lds_sync();
          for (int i = lane; i < nin; i += 64) {
            const int j = key_of<SPLIT>(cg, len, tin[i]);
            atomicAdd(&cw[j >> 1], 1u << ((j & 1) * 16));
          }
          wave_lds_sync();
          int lsum = 0;
#pragma unroll
          for (int i = 0; i < kPer / 2; ++i) {
            const uint32_t word = cw[lane * (kPer / 2) + i];
            cnt[2 * i] = (int)(word & 0xffffu);
            cnt[2 * i + 1] = (int)(word >> 16);
            lsum += cnt[2 * i] + cnt[2 * i + 1];
          }
          const int bsum = __builtin_amdgcn_readlane(wave_incl_scan_dpp(before), 63);
          const int nstart = bsum + wave_incl_scan_dpp(lsum) - lsum;
          if (ix) {
            int k = nstart;
#pragma unroll
            for (int i = 0; i < kPer; ++i)
              for (int c = 0; c < cnt[i] && k < S; ++c) ix[k++] = k0 + lane * kPer + i;
          }
          uint32_t sel = 0;
#pragma unroll
          for (int i = 0; i < kPer; ++i) sel |= (cnt[i] > 0 ? 1u : 0u) << i;
          const int nl = __popc(sel);
          const int incl_n = wave_incl_scan_dpp(nl);
          nsel = __builtin_amdgcn_readlane(incl_n, 63);
          if (nsel > 0) {
            wave_lds_sync();  // every lane is done with the local CDF
            // every key is written; an unselected one goes to the lane's own
            // slot past the list (no branches, no two lanes on one address)
            int pos = incl_n - nl;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
              const bool on = cnt[i] > 0;
              list[on ? pos : SPLIT + lane] = (uint32_t)(lane * kPer + i) | ((uint32_t)cnt[i] << 16);
              pos += on ? 1 : 0;
            }
          }
        } else {
          // systematic / stratified: the number of points below an edge X is a
          // closed-form function of y = X S / Z; a key's count is the
          // difference at its two edges.  y = ylo + a cum, cum the exact local
          // CDF value at the edge, clamped to the split's end yhi; an edge
          // shared with the neighbouring key, lane or split is the same double
          // on both sides (the same operations on the same exact operands), so
          // every point is counted once.  The sequence's last key ends at t = 1.
          const double inv = (double)S / Z;
          const double u0 = p.mode == 2 ? usys : 0.0;
          const double ylo = fma(Olo, inv, -u0), yhi = fma(Ohi, inv, -u0), a = rs * inv;
          auto place = [&](auto sys) {
            // number of points below the right edge of key k (k = -1: the
            // split's left edge), cum the exact local CDF value there
            auto n_at = [&](int k, double cum) -> int {
              const bool end = k >= len - 1;
              const double y = end ? yhi : fmin(fma(cum, a, ylo), yhi);
              int n;
              if constexpr (decltype(sys)::value) {
                n = min(max((int)ceil(y), 0), S);  // t_k = (k + u) / S: ceil(y)
              } else {
                // t_k = (k + u_k) / S: f + [u_f < y - f], f = floor(y)
                const double f = fmin(floor(y), (double)S);
                const uint32_t uf = ug[min((int)f, S - 1)];
                n = (int)f + ((f < (double)S && (double)uf * 0x1.0p-24 < y - f) ? 1 : 0);
              }
              return end && is_last ? S : n;
            };
            // the lane's two edges: points nL .. nR - 1 fall in its keys
            const int nL = n_at(lane * kPer - 1, wt.excl);
            const int nR = n_at(lane * kPer + kPer - 1, wt.excl + wt.lsum);
            // Only lanes with points need their keys' edges.  NSRC = 64 / kPer
            // such source lanes at a time: lane j * kPer + i takes key i of the
            // j-th of them, whose exact CDF value comes from a scan of the
            // weights over its segment of kPer lanes; the source lane's prefix
            // and left-edge count are fetched by a lane permutation.
            constexpr int NSRC = 64 / kPer;
            uint64_t act = __ballot(nR > nL);
            const int jsrc = lane / kPer, i = lane % kPer;
            const uint64_t exu = __builtin_bit_cast(uint64_t, wt.excl);
            while (act != 0ull) {
              int sl = -1;
#pragma unroll
              for (int x = 0; x < NSRC; ++x) {
                const int f = act != 0ull ? __ffsll((unsigned long long)act) - 1 : -1;
                sl = jsrc == x ? f : sl;
                act &= act - 1ull;  // (no effect once empty)
              }
              const bool valid = sl >= 0;
              const int key = (valid ? sl : 0) * kPer + i;
              const uint32_t qk = list[lidx(key)];  // the key's weight
              const double c = seg_scan_exact<kPer>(valid ? (double)qk : 0.0, i);
              const int baddr = (valid ? sl : 0) * 4;
              const uint32_t elo = (uint32_t)__builtin_amdgcn_ds_bpermute(baddr, (int)(uint32_t)exu);
              const uint32_t ehi = (uint32_t)__builtin_amdgcn_ds_bpermute(baddr, (int)(uint32_t)(exu >> 32));
              const double ex = __builtin_bit_cast(double, ((uint64_t)ehi << 32) | elo);
              const int nl0 = __builtin_amdgcn_ds_bpermute(baddr, nL);
              const int nr = n_at(key, ex + c);  // right edge of the key
              const int up = __builtin_amdgcn_update_dpp(0, nr, 0x111, 0xF, 0xF, true);  // right edge of key - 1 (i > 0)
              const int nl = i == 0 ? nl0 : up;
              const int cnt = valid ? nr - nl : 0;
              const uint64_t selm = __ballot(cnt > 0);
              const int pos = nsel + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(selm >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)selm, 0u));
              if (cnt > 0) {
                list[pos] = (uint32_t)key | ((uint32_t)cnt << 16);
                if (ix)
                  for (int x = 0; x < cnt && nl + x < S; ++x) ix[nl + x] = k0 + key;
              }
              nsel += __popcll(selm);
            }
          };
          if (p.mode == 2)
            place(Flag<true>{});
          else
            place(Flag<false>{});
        }

        // 5. gather: each selected value row is read once and weighted by its
        // count (an exact product in fp32); the first kVU rows per lane are
        // requested here
        gt.nsel = nsel;
        if (nsel > 0) {
          wave_lds_sync();
          const int rr = lane / LPR, c = lane % LPR;
#pragma unroll
          for (int u = 0; u < kVU; ++u) {
            const int x = u * RPW + rr;
            gt.ee[u] = x < nsel ? list[x] : 0u;
            gt.vv[u] = x < nsel ? *(const uint4*)(row_of(p.V, it, wb, (int)(gt.ee[u] & 0xffffu)) + c * 8)
                                : make_uint4(0, 0, 0, 0);
          }
        }
  };
  // Deterministic mode: the split's share of head g's estimate, sum over its
  // selected keys of count * V row, is formed exactly (fp16 values are
  // multiples of 2^-24 below 2^16, so every product and partial sum of at most
  // kMaxS points is a multiple of 2^-24 below 2^50: exact in fp64) and added in
  // units of 2^-24 to the head's int64 row, together with a marker 2^52 per
  // element, so integer sums make the total independent of the order the
  // splits arrive in.  Every split adds (its share may be zero), and the
  // group's last split waits until every element carries nsg markers, then
  // writes out = total 2^-24 / S, rounded once to fp32.
  constexpr uint64_t kMarker = 1ull << 52;
  auto tail_exact = [&](const ItemCtx& it, int g, int wb, const Gather& gt) {
        const int nsel = gt.nsel;
        const uint32_t row = (uint32_t)(it.b * p.Hq + it.h0 + g);
        float* scb = score_buf(wb);
        const uint32_t* list = (const uint32_t*)(scb + g * kPad);
        const int r = lane / LPR, c = lane % LPR;
        double a8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a8[e] = 0.0;
        auto add_rows = [&](const uint4 (&vv)[kVU], const uint32_t (&ee)[kVU]) {
#pragma unroll
          for (int u = 0; u < kVU; ++u) {
            const double cf = (double)(ee[u] >> 16);
            float f8[8];
            unpack8(vv[u], f8);
#pragma unroll
            for (int e = 0; e < 8; ++e) a8[e] = fma(cf, (double)f8[e], a8[e]);  // exact
          }
        };
        if (nsel > 0) {
          add_rows(gt.vv, gt.ee);
          for (int i0 = RPW * kVU; i0 < nsel; i0 += RPW * kVU) {
            uint4 vv[kVU];
            uint32_t ee[kVU];
#pragma unroll
            for (int u = 0; u < kVU; ++u) {
              const int i = i0 + u * RPW + r;
              ee[u] = i < nsel ? list[i] : 0u;
              vv[u] = i < nsel ? *(const uint4*)(row_of(p.V, it, wb, (int)(ee[u] & 0xffffu)) + c * 8)
                               : make_uint4(0, 0, 0, 0);
            }
            add_rows(vv, ee);
          }
        }
        // the RPW row slots are summed through LDS (the head's uniform row, free
        // by now) so that lane l ends with features l, l + 64, ...
        double* part = (double*)(uni + g * kUniRow);  // [RPW][D]
        wave_lds_sync();
#pragma unroll
        for (int e = 0; e < 8; ++e) part[r * D + c * 8 + e] = a8[e];
        wave_lds_sync();
        uint64_t* arow = p.ws.acc + (size_t)row * D;
#pragma unroll
        for (int f = 0; f < D / 64; ++f) {
          double v = 0.0;
#pragma unroll
          for (int x = 0; x < RPW; ++x) v += part[x * D + f * 64 + lane];  // exact
          // v 2^24 is an integer below 2^50 in magnitude: adding 1.5 2^52
          // leaves it in the low mantissa bits (two's complement offset)
          const double y = fma(v, 16777216.0, 6755399441055744.0);
          const int64_t units = (int64_t)(__builtin_bit_cast(uint64_t, y) - 0x4338000000000000ull);
          atomic_add_dev(arow + f * 64 + lane, (uint64_t)units + kMarker);
        }
        if (!it.is_last) return;
        // the group's last split: wait for every split's share, then round once
        wait_memory();
        const uint64_t want = (uint64_t)it.nsg;
        uint64_t tot[D / 64];
        uint32_t spins = 0;
        while (true) {
          bool ok = true;
#pragma unroll
          for (int f = 0; f < D / 64; ++f) {
            tot[f] = load_dev(arow + f * 64 + lane);
            ok = ok && ((tot[f] + (kMarker >> 1)) >> 52) == want;
          }
          if (__ballot(!ok) == 0ull) break;
          if (++spins > kSpinLimit) {
            if (lane == 0) atomicOr(p.ws.err, kErrSpinTimeout);
            break;
          }
          __builtin_amdgcn_s_sleep(kPollSleep);
        }
        float* orow = p.out + (size_t)row * D;
#pragma unroll
        for (int f = 0; f < D / 64; ++f) {
          const int64_t units = (int64_t)(tot[f] - want * kMarker);
          orow[f * 64 + lane] = (float)((double)units * 0x1.0p-24 / (double)S);
        }
  };
  auto tail_b = [&](const ItemCtx& it, int g, int wb, const Gather& gt) {
        const int nsel = gt.nsel;
        if (p.det) {
          tail_exact(it, g, wb, gt);
          return;
        }
        if (nsel == 0) return;
        const int b = it.b, hk = it.hk, k0 = it.k0;
        const uint32_t row = (uint32_t)(b * p.Hq + it.h0 + g);
        float* orow = p.out + (size_t)row * D;
        const uint32_t* list = (const uint32_t*)(score_buf(wb) + g * kPad);
        {
          const int r = lane / LPR, c = lane % LPR;
          float a8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) a8[e] = 0.f;
          // rounds past the list (nsel is the same in every lane) are skipped
          auto add_rows = [&](const uint4 (&vv)[kVU], const uint32_t (&ee)[kVU], int i0) {
#pragma unroll
            for (int u = 0; u < kVU; ++u) {
              if (i0 + u * RPW >= nsel) break;
              const float cf = (float)(ee[u] >> 16);
              float f8[8];
              unpack8(vv[u], f8);
#pragma unroll
              for (int e = 0; e < 8; ++e) a8[e] = fmaf(cf, f8[e], a8[e]);
            }
          };
          add_rows(gt.vv, gt.ee, 0);
          for (int i0 = RPW * kVU; i0 < nsel; i0 += RPW * kVU) {
            uint4 vv[kVU];
            uint32_t ee[kVU];
#pragma unroll
            for (int u = 0; u < kVU; ++u) {
              const int i = i0 + u * RPW + r;
              ee[u] = i < nsel ? list[i] : 0u;
              vv[u] = i < nsel ? *(const uint4*)(row_of(p.V, it, wb, (int)(ee[u] & 0xffffu)) + c * 8)
                               : make_uint4(0, 0, 0, 0);
            }
            add_rows(vv, ee, i0);
          }
          // Sum the RPW row slots in registers (reduce-scatter).  Lane (r, c)
          // holds features c*8 .. c*8+7 of row slot r.  A swap of the wave's
          // halves pairs feature e with e + 4 (the lower half keeps the sums of
          // 0..3, the upper those of 4..7) and a swap of odd and even rows of
          // 16 pairs the remaining j with j + 2: lane (r, c) then holds the
          // totals of features c*8 + 2r and c*8 + 2r + 1 (D = 128).  For D = 64
          // (rows of 8 lanes) a rotation adds the two halves of each row of 16,
          // and lane (r, c) keeps feature c*8 + r.  For D = 128 a lane
          // permutation gives lane l features l and 64 + l, so that each atomic
          // instruction covers 64 consecutive floats (two cache lines, not four:
          // the splits of a head all add into the same row).
          float h4[4], h2[2];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(a8[e]), __float_as_uint(a8[e + 4]), false, false);
            h4[e] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(h4[e]), __float_as_uint(h4[e + 2]), false, false);
            h2[e] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
          }
          const float inv_s = 1.0f / (float)S;  // exact for a power of two S, else one more rounding
          if constexpr (D == 128) {
            // lane l takes features l and 64 + l: feature F = c*8 + 2R + e sits in lane 16R + c, value e
            const int e = lane & 1, R = (lane & 7) >> 1, cc = lane >> 3;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const int src_lane = 16 * R + cc + 8 * f;
              const float v0 = __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane * 4, __float_as_int(h2[0])));
              const float v1 = __int_as_float(__builtin_amdgcn_ds_bpermute(src_lane * 4, __float_as_int(h2[1])));
              atomic_add_dev(orow + f * 64 + lane, (e ? v1 : v0) * inv_s);
            }
          } else {
            static_assert(D == 64, "head dimension");
            const float s0 = h2[0] + dpp_row_ror<0x128>(h2[0]);
            const float s1 = h2[1] + dpp_row_ror<0x128>(h2[1]);
            atomic_add_dev(orow + c * 8 + r, ((r & 1) ? s1 : s0) * inv_s);
          }
        }
  };

  // ---- stream one split, publish its statistics (all waves) -----------------
  // K loads per lane and buffer of the row-major score stages: two workgroups
  // per CU take half (the CU still has 16 KiB per wave in flight, and the
  // registers saved avoid spills)
  constexpr int kRowLB = OCC == 2 ? (G > kWaves ? 4 : 8) : 16;
  // One item per workgroup, fp16 or fp8 row-major cache: the query and the
  // first K rows are requested before the sequence length has arrived (the
  // rows are clamped to the K block, not to the length), so the stream
  // starts one round trip earlier.
  constexpr bool kEarlyRows = (KIND == kKeyF16 || (KIND == kKeyF8 && fp8_supported<D, G>())) && !LOOP;
  using EarlyRows = typename std::conditional<KIND == kKeyF8, RowScoreF8<D, G, kRowLB, SPLIT>,
                                              RowScore<D, G, kRowLB, SPLIT>>::type;
  auto start_item = [&](const ItemCtx& it, float* scb, int wb, bool finish_now, EarlyRows& early) {
    if constexpr (kEarlyRows)
      if (!it.active) early.drop();
    if (!it.valid) {
      if (it.s == 0) {  // invalid sequence length: NaN output, indices -1
        for (int i = tid; i < G * D; i += kThreads) p.out[(size_t)(it.b * p.Hq + it.h0) * D + i] = __builtin_nanf("");
        if (p.idx_out)
          for (int i = tid; i < G * S; i += kThreads) p.idx_out[(size_t)(it.b * p.Hq + it.h0) * S + i] = -1;
      }
      return;
    }
    if (!it.active) return;
    // split 0 clears the group's output rows, each wave the rows of the
    // heads it owns after the score stage (its own wait before publishing
    // covers them); every split adds into a row only after it has seen
    // split 0's statistics for that head
    if (it.s == 0)
      for (int g = w; g < G; g += kWaves) {
        const size_t row = (size_t)(it.b * p.Hq + it.h0 + g) * D;
        if (p.det) {
          for (int i = lane; i < D; i += 64) store_dev(p.ws.acc + row + i, 0ull);
        } else {
          for (int i = lane; i < D; i += 64) store_dev(p.out + row + i, 0.f);
        }
      }

    // ---- score stage: all keys of the split, G query heads ----------------
    float mx[G];
    if constexpr (BERN) {
      bernoulli_load<BUDGET>(p, it.group, sh, binfo, bwt, bwt2);
      score_bernoulli<D, G, BUDGET>(p, it.b, it.hk, it.k0, it.len, scb, mx, sh, binfo, bwt, bwt2);
    } else if constexpr (KIND == kKeyF8) {
      if constexpr (kEarlyRows)
        early.run(p, it.len, scb, mx);
      else
        score_rowmajor_f8<D, G, kRowLB>(p, it.b, it.hk, it.k0, it.len, scb, mx);
    } else {
      if constexpr (PAGED) {
        // the split's block entries, checked against the pool
        const int nbl = (it.len + (1 << p.lg_block) - 1) >> p.lg_block;
        if (tid < nbl) {
          int e = p.block_table[(size_t)it.b * (p.max_n_k >> p.lg_block) + (it.k0 >> p.lg_block) + tid];
          if (e < 0 || e >= p.num_blocks) {
            atomicOr(p.ws.err, kErrBlockTable);
            e = 0;
          }
          pblk[wb][tid] = e;
        }
        lds_barrier();
      }
      if constexpr (PAGED)
        score_rowmajor_rows<D, G, kRowLB>(p, it.b, it.hk, it.len, scb, mx,
                                          [&](int j) { return row_of(p.K, it, wb, j); });
      else if constexpr (kEarlyRows)
        early.run(p, it.len, scb, mx);
      else
        score_rowmajor<D, G, kRowLB, SPLIT>(p, it.b, it.hk, it.k0, it.len, scb, mx);
    }
    if constexpr (BERN) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m = wave_max(mx[g]);
        if (lane == 0) sh.wmax[wb][w][g] = m;
      }
    } else {
      // the row-major stages leave head (lane mod G)'s running maximum in each
      // lane (and -inf for the other heads): one value per head and row of 16
      // lanes, combined by the readers
      float m = mx[0];
#pragma unroll
      for (int g = 1; g < G; ++g) m = fmaxf(m, mx[g]);
      m = row_max_mod<G>(m);
      if ((lane & 15) < G) sh.wmax[wb][w * 4 + (lane >> 4)][lane & 15] = m;
    }
    if (w == 0 && !tagged) {
      uint64_t c = tid < kLaunchCounters ? lc : 0ull;
      asm volatile("" : "+v"(c));  // keeps the wait for the counter reads here, after the stream
      uint64_t sum = 0ull;
#pragma unroll
      for (int i = 0; i < kLaunchCounters; ++i) sum += readlane_u64(c, i);
      if (tid == 0) sh.epoch = tag_of(sum);
    }
    tagged = true;
    lds_barrier();
    if (p.scores_out) {
      write_scores<G, SPLIT>(p, it.b, it.hk, it.k0, it.len, scb);
      __syncthreads();
    }
    // ---- from here on, wave g owns query head g ----------------------------
    for (int g = w; g < G; g += kWaves) {
      Weights wt;
      weights(it, g, scb, wb, wt);
      publish(it, g, wt);
      if (finish_now) {
        Gather gt;
        tail_a(it, g, scb, wb, wt, gt, false);
        tail_b(it, g, wb, gt);
      } else {
        stash_weights(g, scb, wt);
      }
    }
  };

  if constexpr (!LOOP) {
    EarlyRows early;
    const ItemCtx it = describe((int)blockIdx.x, [&](const ItemCtx& c) {
      if constexpr (kEarlyRows) early.begin(p, c.b, c.hk, c.k0, min(SPLIT, p.max_n_k - c.k0));
    });
    start_item(it, score_buf(0), 0, true, early);
  } else {
    // Only valid splits are items, numbered sequence by sequence: sequence b
    // has H_kv * nsg_b of them (nsg_b = ceil(n_k[b] / SPLIT) for a valid
    // length, none otherwise).  Workgroup x takes items x, x + grid,
    // x + 2 grid, ... (no shared counter, no skipped splits).  The splits of
    // a group are consecutive items, so with nsg <= grid they fall in at most
    // two consecutive rounds; every workgroup publishes its item of round r
    // before it waits for any item of round r or later, so the waits end.
    if (tid < kLaunchCounters && !tagged) lc = load_dev(p.ws.launches + tid * kLaunchStride);
    // sequences with an invalid length: NaN outputs, indices -1
    for (int bq = blockIdx.x; bq < p.B; bq += p.grid) {
      const int n = p.n_k[bq];
      if (n >= 1 && n <= p.max_n_k) continue;
      for (int i = tid; i < p.Hq * D; i += kThreads) p.out[(size_t)bq * p.Hq * D + i] = __builtin_nanf("");
      if (p.idx_out)
        for (int i = tid; i < p.Hq * S; i += kThreads) p.idx_out[(size_t)bq * p.Hq * S + i] = -1;
    }
    // lane l of every wave keeps the length of sequence l of the first 64
    const int nk0 = lane < p.B ? p.n_k[lane] : 0;
    // item t -> (sequence, KV head, split); false when t is past the last item
    auto find = [&](int t, ItemCtx& it) -> bool {
      int carry = 0;
      for (int c0 = 0; c0 < p.B; c0 += 64) {
        const int bq = c0 + lane;
        const int n = c0 == 0 ? nk0 : (bq < p.B ? p.n_k[bq] : 0);
        const int nsgq = (n >= 1 && n <= p.max_n_k) ? (n + SPLIT - 1) / SPLIT : 0;
        const int cnt = nsgq * p.Hkv;
        const int incl = wave_incl_scan_dpp(cnt) + carry;
        const uint64_t hit = __ballot(incl > t);
        if (hit != 0ull) {
          const int l = __ffsll((unsigned long long)hit) - 1;
          const int j = t - __builtin_amdgcn_readlane(incl - cnt, l);
          const int nb = __builtin_amdgcn_readlane(n, l), nsgb = __builtin_amdgcn_readlane(nsgq, l);
          it.b = c0 + l;
          it.hk = j / nsgb;
          it.s = j % nsgb;
          it.h0 = it.hk * G;
          it.group = it.b * p.Hkv + it.hk;
          it.valid = true;
          it.active = true;
          it.nsg = nsgb;
          it.k0 = it.s * SPLIT;
          it.len = min(SPLIT, nb - it.k0);
          it.is_last = it.s == nsgb - 1;
          return true;
        }
        carry = __builtin_amdgcn_readlane(incl, 63);
      }
      return false;
    };
    ItemCtx prev{};  // nothing to finish yet (active = false)
    int cb = 0;
    for (int t = blockIdx.x;; t += p.grid) {
      ItemCtx cur{};
      const bool have = find(t, cur);
      EarlyRows unused;  // (the persistent variant scores through score_rowmajor)
      if (have) start_item(cur, score_buf(cb), cb, false, unused);
      if (prev.active)  // the previous item's statistics are published by now, or soon
        for (int g = w; g < G; g += kWaves) {
          Weights wt;
          Gather gt;
          reload_weights(g, score_buf(cb ^ 1), wt);
          tail_a(prev, g, score_buf(cb ^ 1), cb ^ 1, wt, gt, true);
          tail_b(prev, g, cb ^ 1, gt);
        }
      if (!have) break;
      lds_barrier();  // every wave is done with the buffer the next item overwrites
      prev = cur;
      cb ^= 1;
    }
  }
  // ---- a workgroup that scored nothing still adds its share ----------------
  // (the amount is computed from the value read, so the add follows the read)
  if (tid == 0 && !counted)
    atomic_add_noret(p.ws.launches + (blockIdx.x % kLaunchCounters) * kLaunchStride, lc == ~0ull ? 0ull : my_add);
}

// The one-item variant with two workgroups per CU asks for 56 KiB of LDS so
// that no more than two of its workgroups share a CU (three would need more
// than the CU's 160 KiB): the grid then spreads over every CU instead of
// stacking up to four workgroups (its register use would allow that) on some.
constexpr size_t kTwoPerCuLds = 56 * 1024;

template <int D, int G, int VAR, int SPLIT>
size_t lds_bytes() {
  const size_t b = Lds<D, G, VAR == kPersistent ? 2 : 1, SPLIT>::bytes;
  return VAR == kOneItemTwo && b < kTwoPerCuLds ? kTwoPerCuLds : b;
}

template <int D, int G, int KIND, int VAR, int SPLIT>
int capacity_t() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  auto fn = decode_kernel<D, G, KIND, VAR, SPLIT>;
  const size_t lds = lds_bytes<D, G, VAR, SPLIT>();
  (void)hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess) return 0;
  return per_cu * cus;
}

template <int D, int G, int KIND, int VAR, int SPLIT>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const size_t lds = lds_bytes<D, G, VAR, SPLIT>();
  hipLaunchKernelGGL((decode_kernel<D, G, KIND, VAR, SPLIT>), dim3(p.grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

// (D, G, key kind, variant, split) combinations that are built: the fp8 score
// stage needs G <= D / 16; 512-key splits exist for the plain fp16 cache with
// one item per workgroup, two workgroups per CU.
template <int D, int G, int KIND, int VAR, int SPLIT>
constexpr bool built() {
  if (KIND == kKeyF8 && !fp8_supported<D, G>()) return false;
  if (SPLIT == 512) return KIND == kKeyF16 && VAR == kOneItemTwo;
  return VAR != kOneItemTwo;
}

template <int KIND, int VAR, int SPLIT>
hipError_t dispatch(const DecodeParams& p, hipStream_t stream) {
#define SANTA_CASE(DD, GG)                                                                     \
  if constexpr (built<DD, GG, KIND, VAR, SPLIT>())                                             \
    if (p.D == DD && p.G == GG) return launch_t<DD, GG, KIND, VAR, SPLIT>(p, stream);
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return hipErrorInvalidValue;
}

template <int KIND, int VAR, int SPLIT>
int capacity(int D, int G) {
#define SANTA_CASE(DD, GG)                                                                     \
  if constexpr (built<DD, GG, KIND, VAR, SPLIT>())                                             \
    if (D == DD && G == GG) return capacity_t<DD, GG, KIND, VAR, SPLIT>();
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return 0;
}

template <int VAR, int SPLIT>
int capacity_kind(int D, int G, int key_kind) {
  if (key_kind == kKeyBernoulli) return capacity<kKeyBernoulli, VAR, SPLIT>(D, G);
  if (key_kind == kKeyBernoulliBudget) return capacity<kKeyBernoulliBudget, VAR, SPLIT>(D, G);
  if (key_kind == kKeyF8) return capacity<kKeyF8, VAR, SPLIT>(D, G);
  if (key_kind == kKeyF16Paged) return capacity<kKeyF16Paged, VAR, SPLIT>(D, G);
  return capacity<kKeyF16, VAR, SPLIT>(D, G);
}

template <int VAR, int SPLIT>
hipError_t dispatch_kind(const DecodeParams& p, int key_kind, hipStream_t stream) {
  if (key_kind == kKeyBernoulli) return dispatch<kKeyBernoulli, VAR, SPLIT>(p, stream);
  if (key_kind == kKeyBernoulliBudget) return dispatch<kKeyBernoulliBudget, VAR, SPLIT>(p, stream);
  if (key_kind == kKeyF8) return dispatch<kKeyF8, VAR, SPLIT>(p, stream);
  if (key_kind == kKeyF16Paged) return dispatch<kKeyF16Paged, VAR, SPLIT>(p, stream);
  return dispatch<kKeyF16, VAR, SPLIT>(p, stream);
}

}  // namespace

hipError_t launch_bernoulli_prep(const DecodeParams& p, int key_kind, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.Hkv)), block(kThreads);
#define SANTA_CASE(DD, GG)                                                                                   \
  if (p.D == DD && p.G == GG) {                                                                             \
    if (key_kind == kKeyBernoulliBudget)                                                                    \
      hipLaunchKernelGGL((bernoulli_prep<DD, GG, true>), grid, block, 0, stream, p);                        \
    else                                                                                                    \
      hipLaunchKernelGGL((bernoulli_prep<DD, GG, false>), grid, block, 0, stream, p);                       \
    return hipGetLastError();                                                                               \
  }
  SANTA_CASE(64, 1) SANTA_CASE(64, 2) SANTA_CASE(64, 4) SANTA_CASE(64, 8)
  SANTA_CASE(128, 1) SANTA_CASE(128, 2) SANTA_CASE(128, 4) SANTA_CASE(128, 8)
#undef SANTA_CASE
  return hipErrorInvalidValue;
}

int decode_capacity(int D, int G, int key_kind, int variant, int split) {
  if (split == 512) return variant == kOneItemTwo ? capacity_kind<kOneItemTwo, 512>(D, G, key_kind) : 0;
  if (variant == kPersistent) return capacity_kind<kPersistent, kSplit>(D, G, key_kind);
  return variant == kOneItem ? capacity_kind<kOneItem, kSplit>(D, G, key_kind) : 0;
}

hipError_t launch_decode(const DecodeParams& p, int key_kind, hipStream_t stream) {
  if (p.split == 512) {
    if (p.occ == kOneItemTwo) return dispatch_kind<kOneItemTwo, 512>(p, key_kind, stream);
    return hipErrorInvalidValue;
  }
  if (p.occ == kPersistent) return dispatch_kind<kPersistent, kSplit>(p, key_kind, stream);
  if (p.occ == kOneItem) return dispatch_kind<kOneItem, kSplit>(p, key_kind, stream);
  return hipErrorInvalidValue;
}

}  // namespace santa
