// Device helpers shared by the libsanta kernels (gfx950, wave64).
//
// Nothing here is specific to one kernel: the Philox4x32-10 generator, fp16
// row-slice loads, DPP cross-lane moves, wave reductions/scans and the
// agent-scope atomics used for the cross-workgroup hand-offs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace santa {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11).  Round: 32x32->64-bit products of c0 and c2 with the
// two round multipliers, output (hi1^c1^k0, lo1, hi0^c3^k1, lo0); the key is
// bumped by the two Weyl constants between rounds; ten rounds.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
  constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
  constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kWeylA;
      k1 += kWeylB;
    }
    const uint32_t lo_a = kMulA * c.x, hi_a = __umulhi(kMulA, c.x);
    const uint32_t lo_b = kMulB * c.z, hi_b = __umulhi(kMulB, c.z);
    c = make_uint4(hi_b ^ c.y ^ k0, lo_b, hi_a ^ c.w ^ k1, lo_a);
  }
  return c;
}

// Stream tags (ASCII of a four-letter name), one stream per use.
constexpr uint32_t kTagSystematic = 0x53595354u;  // 'SYST'
constexpr uint32_t kTagStratified = 0x53545254u;  // 'STRT'
constexpr uint32_t kTagIid = 0x49494420u;         // 'IID '
constexpr uint32_t kTagBernoulli = 0x4245524Eu;   // 'BERN'

// Block `blk` of stream (seed, row, tag): words 4*blk .. 4*blk+3.
__device__ __forceinline__ uint4 stream_block(uint64_t seed, uint32_t row, uint32_t tag, uint32_t blk) {
  return philox4x32_10(make_uint4(blk, row, tag, 0u), (uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32));
}

__device__ __forceinline__ uint32_t word_of(uint4 w, int e) {
  return e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
}

// 24-bit integer behind a uniform: u = (x >> 8) * 2^-24 exactly.
__device__ __forceinline__ uint32_t uniform_bits(uint32_t x) { return x >> 8; }
__device__ __forceinline__ double uniform_f64(uint32_t x) { return (double)(x >> 8) * 0x1.0p-24; }

// ---------------------------------------------------------------------------
// fp16 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }

// 8-element fp16 dot product accumulated in fp32 (v_dot2 on gfx950).
__device__ __forceinline__ float dot8(uint4 a, uint4 b) {
  float acc = 0.f;
  acc = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(b.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(b.w), acc, false);
  return acc;
}

__device__ __forceinline__ void unpack8(uint4 v, float* f) {
  half2v h;
  h = as_h2(v.x); f[0] = (float)h.x; f[1] = (float)h.y;
  h = as_h2(v.y); f[2] = (float)h.x; f[3] = (float)h.y;
  h = as_h2(v.z); f[4] = (float)h.x; f[5] = (float)h.y;
  h = as_h2(v.w); f[6] = (float)h.x; f[7] = (float)h.y;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: the data is read once).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// DPP lane exchanges inside a 16-lane row.
// ---------------------------------------------------------------------------
enum DppCtrl : int {
  kDppXor1 = 0xB1,          // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,          // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,   // lane ^ 7 inside each group of 8
  kDppRor8 = 0x128,         // lane ^ 8 inside each row of 16
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Reduce-scatter across the LPR lanes of a key row.  On entry every lane holds
// NV = LPR partial sums v[0..NV); on exit lane (lane % LPR) holds in v[0] the
// full sum of combination index (lane % LPR).  Partner lanes are paired with
// the masks 8, 7, 2, 1 (LPR = 16), 7, 2, 1 (LPR = 8) or 2, 1 (LPR = 4); the
// half kept by a lane is chosen by one bit of its lane id that differs between
// partners.
template <int LPR>
__device__ __forceinline__ void row_reduce_scatter(float* v, int lane) {
  static_assert(LPR == 4 || LPR == 8 || LPR == 16, "row width");
  if constexpr (LPR == 16) {
    const bool hi = (lane >> 3) & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float send = hi ? v[i] : v[i + 8];
      float keep = hi ? v[i + 8] : v[i];
      v[i] = keep + dpp<kDppRor8>(send);
    }
  }
  if constexpr (LPR >= 8) {
    const bool hi = (lane >> 2) & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float send = hi ? v[i] : v[i + 4];
      float keep = hi ? v[i + 4] : v[i];
      v[i] = keep + dpp<kDppHalfMirror>(send);
    }
  }
  {
    const bool hi = (lane >> 1) & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float send = hi ? v[i] : v[i + 2];
      float keep = hi ? v[i + 2] : v[i];
      v[i] = keep + dpp<kDppXor2>(send);
    }
  }
  {
    const bool hi = lane & 1;
    float send = hi ? v[0] : v[1];
    float keep = hi ? v[1] : v[0];
    v[0] = keep + dpp<kDppXor1>(send);
  }
}

// ---------------------------------------------------------------------------
// Wave-level reductions and scans (64 lanes).
// ---------------------------------------------------------------------------
// DPP move of a 64-bit value (two 32-bit halves); lanes without a source, or
// outside ROW_MASK, read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, ROW_MASK, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, ROW_MASK, 0xF, true);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum over the wave: shifts by 1, 2, 4, 8 inside each row
// of 16 lanes, then the last lane of row 0 is added to row 1 (and of row 2 to
// row 3), then the last lane of row 1 to rows 2 and 3.  Integer, so exact.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  v += dpp_u64<0x111, 0xF>(v);  // row_shr:1
  v += dpp_u64<0x112, 0xF>(v);  // row_shr:2
  v += dpp_u64<0x114, 0xF>(v);  // row_shr:4
  v += dpp_u64<0x118, 0xF>(v);  // row_shr:8
  v += dpp_u64<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_u64<0x143, 0xC>(v);  // row_bcast:31 into rows 2, 3
  return v;
}

// The same scan on doubles that hold integers below 2^53: every partial sum
// is exact, so the result does not depend on the order of the additions.
__device__ __forceinline__ double wave_incl_scan_exact(double v) {
  v += __builtin_bit_cast(double, dpp_u64<0x111, 0xF>(__builtin_bit_cast(uint64_t, v)));
  v += __builtin_bit_cast(double, dpp_u64<0x112, 0xF>(__builtin_bit_cast(uint64_t, v)));
  v += __builtin_bit_cast(double, dpp_u64<0x114, 0xF>(__builtin_bit_cast(uint64_t, v)));
  v += __builtin_bit_cast(double, dpp_u64<0x118, 0xF>(__builtin_bit_cast(uint64_t, v)));
  v += __builtin_bit_cast(double, dpp_u64<0x142, 0xA>(__builtin_bit_cast(uint64_t, v)));
  v += __builtin_bit_cast(double, dpp_u64<0x143, 0xC>(__builtin_bit_cast(uint64_t, v)));
  return v;
}

__device__ __forceinline__ uint64_t wave_bcast_u64(uint64_t v, int lane_src) {
  const uint32_t lo = __shfl((int)(uint32_t)v, lane_src, 64);
  const uint32_t hi = __shfl((int)(uint32_t)(v >> 32), lane_src, 64);
  return ((uint64_t)hi << 32) | lo;
}
// Maximum over the 64 lanes of a wave, returned in every lane: DPP row
// shifts (empty sources read -inf) and row broadcasts leave the maximum in
// lane 63, which is then read as a scalar.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max_step(float v) {
  const float other = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -INFINITY), __builtin_bit_cast(int, v), CTRL,
                                         ROW_MASK, 0xF, false));
  return fmaxf(v, other);
}
__device__ __forceinline__ float wave_max(float v) {
  v = dpp_max_step<0x111, 0xF>(v);  // row_shr:1
  v = dpp_max_step<0x112, 0xF>(v);  // row_shr:2
  v = dpp_max_step<0x114, 0xF>(v);  // row_shr:4
  v = dpp_max_step<0x118, 0xF>(v);  // row_shr:8
  v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15
  v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Maximum over the lanes of this lane's row of 16 that are congruent to it
// modulo G (G a power of two, at most 8), in every lane: rotations of the row
// by G, 2G, .., 8.
template <int CTRL>
__device__ __forceinline__ float dpp_row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int G>
__device__ __forceinline__ float row_max_mod(float v) {
  static_assert(G >= 1 && G <= 8 && (G & (G - 1)) == 0, "G is a power of two up to 8");
  if constexpr (G <= 1) v = fmaxf(v, dpp_row_ror<0x121>(v));  // row_ror:1
  if constexpr (G <= 2) v = fmaxf(v, dpp_row_ror<0x122>(v));  // row_ror:2
  if constexpr (G <= 4) v = fmaxf(v, dpp_row_ror<0x124>(v));  // row_ror:4
  return fmaxf(v, dpp_row_ror<0x128>(v));                     // row_ror:8
}

// Inclusive prefix sum of 32-bit integers over the wave (same DPP pattern).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += dpp_i32<0x111, 0xF>(v);
  v += dpp_i32<0x112, 0xF>(v);
  v += dpp_i32<0x114, 0xF>(v);
  v += dpp_i32<0x118, 0xF>(v);
  v += dpp_i32<0x142, 0xA>(v);
  v += dpp_i32<0x143, 0xC>(v);
  return v;
}

__device__ __forceinline__ float wave_max_masked(float x, int first_mask) {
  for (int m = first_mask; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
  return x;
}

__device__ __forceinline__ double wave_incl_scan_f64(double x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    double y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_incl_scan_i32(int x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

// ---------------------------------------------------------------------------
// Hand-offs between workgroups.
//
// On gfx950 an agent-scope release or acquire fence writes back or
// invalidates the whole L2 of the XCD (the L2s of the 8 XCDs are not
// coherent with each other for ordinary loads and stores), which costs
// microseconds per fence.  Data exchanged between workgroups therefore never
// goes through ordinary stores plus fences: it is written with device-scope
// stores (sc1, written through to the device coherence point) and read with
// device-scope loads (sc1, never served from a stale L2 line).  A producer
// waits until its device-scope stores are acknowledged (s_waitcnt on all
// outstanding memory operations) before it bumps the arrival counter with an
// atomic; a consumer issues its device-scope loads only after it has seen the
// counter value, so it reads what the producers wrote.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t atomic_add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_add_noret(uint64_t* p, uint64_t v) {
  (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-scope 64-bit integer add without return (global_atomic_add_x2).
__device__ __forceinline__ void atomic_add_dev(uint64_t* p, uint64_t v) {
  (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-scope float add without return (global_atomic_add_f32).
__device__ __forceinline__ void atomic_add_dev(float* p, float v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_dev(const float2* p) {
  const uint64_t v = __hip_atomic_load((uint64_t*)const_cast<float2*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(float2, v);
}
__device__ __forceinline__ void store_dev(float2* p, float2 v) {
  __hip_atomic_store((uint64_t*)p, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte read that bypasses the caches between this CU and the device's
// coherence point (global_load_dwordx4 sc0 sc1), for polling a 16-byte slot
// whose halves another workgroup writes with device-scope stores: each half
// is read as one value, and a reader that sees a half not yet written retries.
__device__ __forceinline__ u32x4 load_dev16(const void* p) {
  return *(const volatile __attribute__((address_space(1))) u32x4*)p;
}
// Workgroup barrier that orders LDS accesses only: global loads and stores
// in flight stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Wait until every memory operation this wave has issued has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0); }

}  // namespace santa
