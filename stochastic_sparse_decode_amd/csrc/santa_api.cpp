// C-ABI layer of libsanta: argument checks, workspace carving, launch shape.
// Declarations and the meaning of every argument: include/santa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "santa.h"
#include "launch.h"

namespace {

using santa::DecodeParams;
using santa::Workspace;

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool problem_ok(const santa_problem* p) {
  if (!p) return false;
  if (p->batch < 1 || p->num_kv_heads < 1 || p->num_q_heads < 1 || p->max_n_k < 1) return false;
  if (p->num_q_heads % p->num_kv_heads != 0) return false;
  if (!std::isfinite(p->scale)) return false;
  const long long groups = (long long)p->batch * p->num_kv_heads;
  const long long ns = ((long long)p->max_n_k + santa::kSplit - 1) / santa::kSplit;
  if (groups * ns > (1ll << 30)) return false;
  if ((long long)p->batch * p->num_q_heads > (1ll << 30)) return false;
  return true;
}

int group_size(const santa_problem* p) { return p->num_q_heads / p->num_kv_heads; }

bool supported(const santa_problem* p) {
  const int G = group_size(p);
  if ((p->flags & ~SANTA_DETERMINISTIC) != 0u) return false;
  return (p->head_dim == 64 || p->head_dim == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

// Workspace layout: a 1 KiB header (error bits, the dense kernel's work
// counter, the launch counters), a 64 KiB region of the dense kernel's arrival
// counters, then the data of the call in two parts:
//  - tagged words, from the start of the data area: the sampling kernel's
//    statistics slots, or the dense kernel's records when its splits exchange
//    them.  A reader accepts such a word only if it carries this launch's
//    tag, and words written by earlier launches carry earlier tags;
//  - untagged data, at the end of the buffer: the exact output sums of the
//    deterministic mode, the Gumbel-max winners, the prepared Bernoulli
//    queries, or the dense kernel's float records.  They are written (or
//    cleared) before they are read in every call.
// The header's work counter and the arrival counters must be zero when a
// launch starts (every dense launch leaves them at zero; the caller zero-fills
// a new buffer), and no data region overlaps them.  santa_workspace_bytes(P)
// leaves room for the larger tagged part and the larger untagged part of P's
// calls of either kind.  Every part grows with each dimension of the problem
// and with S, so in a buffer of that size (passed with the same size every
// time) the tagged words of any call whose problem is no larger never overlap
// the untagged data of another: stale untagged data, whose bits are
// arbitrary, can never be taken for a slot of this launch.
constexpr size_t kCounterBytes = (size_t)santa::kMaxDenseGroups * sizeof(uint32_t);
constexpr size_t kHeaderBytes = 1024;  // error bits, work counter, kLaunchCounters launch counters (one per 128 bytes)

struct Layout {
  size_t xrec, partial, stats, acc, win, bern;
  size_t tagged() const { return xrec > stats ? xrec : stats; }
  size_t untagged() const { return partial > acc + win + bern ? partial : acc + win + bern; }
  size_t dense_total() const { return kHeaderBytes + kCounterBytes + xrec + partial; }
  size_t sampling_total() const { return kHeaderBytes + kCounterBytes + stats + acc + win + bern; }
  size_t total() const { return kHeaderBytes + kCounterBytes + tagged() + untagged(); }
};

// S: the sample count of the call (the Gumbel-max draws keep one winner per
// query head and draw).
Layout layout_of(const santa_problem* p, int32_t S) {
  Layout L{};
  const size_t groups = (size_t)p->batch * p->num_kv_heads;
  const size_t G = (size_t)group_size(p), D = (size_t)p->head_dim;
  const size_t ns_min = ((size_t)p->max_n_k + santa::kMinSplit - 1) / santa::kMinSplit;
  L.xrec = round_up(groups * ns_min * G * (D + 2) * sizeof(uint64_t));  // at either split length
  L.partial = round_up(groups * ns_min * G * (D + 2) * sizeof(float));
  L.stats = round_up(groups * ns_min * G * (size_t)santa::slot_words_for(groups * ns_min * G) * sizeof(uint64_t));
  L.acc = round_up(groups * G * D * sizeof(uint64_t));
  L.win = round_up((size_t)p->batch * p->num_q_heads * (size_t)S * sizeof(uint64_t));
  L.bern = round_up(groups * santa::kBernRecord * 16);
  return L;
}

// ws_bytes: the buffer's size as passed (the untagged part ends there).  err,
// if not null, takes the place of the header's error word.
Workspace carve(void* base, size_t ws_bytes, const santa_problem* p, int32_t S, bool dense,
                uint32_t* err = nullptr) {
  unsigned char* b = (unsigned char*)base;
  const Layout L = layout_of(p, S);
  Workspace w{};
  w.err = err ? err : (uint32_t*)b;
  w.work_ctr = (uint32_t*)b + 1;
  w.launches = (uint64_t*)(b + 128);  // counter i at launches + i * kLaunchStride
  w.arrive = (uint32_t*)(b + kHeaderBytes);
  unsigned char* x = b + kHeaderBytes + kCounterBytes;
  unsigned char* end = b + ws_bytes / kAlign * kAlign;
  if (dense) {
    w.xrec = (uint64_t*)x;
    w.partial = (float*)(end - L.partial);
  } else {
    w.stats = (uint64_t*)x;
    w.acc = (uint64_t*)(end - (L.acc + L.win + L.bern));
    w.win = (uint64_t*)(end - (L.win + L.bern));
    w.bern = (uint4*)(end - L.bern);
  }
  return w;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// Resident-workgroup capacity per (device, kernel variant), computed once.
constexpr int kMaxDevices = 64;
constexpr int kVariants = 2 /*D*/ * 4 /*G*/ * 6 /*kernel*/ * 4 /*variant: dense, 1, 2, 3*/ * 2 /*split*/;
std::mutex g_cap_mutex;
int g_cap[kMaxDevices][kVariants];

int variant_index(int D, int G, int kind, int occ, int split) {
  const int di = D == 128 ? 1 : 0;
  const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
  return (((kind * 2 + di) * 4 + gi) * 4 + (occ & 3)) * 2 + (split == santa::kSplit ? 0 : 1);
}

int key_kind(int op) {
  switch (op) {
    case santa::kOpBernoulli: return santa::kKeyBernoulli;
    case santa::kOpDecodeF8: return santa::kKeyF8;
    case santa::kOpDecodePaged: return santa::kKeyF16Paged;
    case santa::kOpBernoulliBudget: return santa::kKeyBernoulliBudget;
    default: return santa::kKeyF16;
  }
}

struct Paging {
  const int32_t* block_table = nullptr;
  int lg_block = 0, num_blocks = 0;
};

// Compute units of the current device (0 on failure), computed once per device.
int g_cus[kMaxDevices];
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(g_cap_mutex);
  if (g_cus[dev] == 0 &&
      hipDeviceGetAttribute(&g_cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    g_cus[dev] = 0;
  return g_cus[dev];
}

int capacity(int D, int G, int kind, int occ, int split = santa::kSplit) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(g_cap_mutex);
  int& slot = g_cap[dev][variant_index(D, G, kind, kind == santa::kOpDense ? 0 : occ, split)];
  if (slot == 0) {
    slot = kind == santa::kOpDense ? santa::dense_capacity(D, G)
                                   : santa::decode_capacity(D, G, key_kind(kind), occ, split);
  }
  return slot;
}

int common_checks(const santa_problem* p, const void* q, const void* K, const void* V, const int32_t* n_k,
                  const float* out, const void* ws, size_t ws_bytes, bool dense, int32_t S = 1) {
  if (!p) return SANTA_ERR_NULL;
  if (!q || !K || !V || !n_k || !out) return SANTA_ERR_NULL;
  if (!problem_ok(p)) return SANTA_ERR_SHAPE;
  if (!supported(p)) return SANTA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 4) || !aligned(n_k, 4))
    return SANTA_ERR_ALIGN;
  const Layout L = layout_of(p, S);
  const size_t need = dense ? L.dense_total() : L.sampling_total();
  if (!ws || ws_bytes / kAlign * kAlign < need || !aligned(ws, kAlign)) return SANTA_ERR_WORKSPACE;
  return SANTA_OK;
}

DecodeParams base_params(const santa_problem* p, const void* q, const void* K, const void* V,
                         const int32_t* n_k, float* out, void* ws, size_t ws_bytes, int32_t S, bool dense,
                         uint32_t* err = nullptr) {
  DecodeParams d{};
  d.q = q;
  d.K = K;
  d.V = V;
  d.n_k = n_k;
  d.out = out;
  d.B = p->batch;
  d.Hq = p->num_q_heads;
  d.Hkv = p->num_kv_heads;
  d.D = p->head_dim;
  d.G = group_size(p);
  d.max_n_k = p->max_n_k;
  d.scale = p->scale;
  d.ns = (p->max_n_k + santa::kSplit - 1) / santa::kSplit;
  d.total_items = p->batch * p->num_kv_heads * d.ns;
  d.ws = carve(ws, ws_bytes, p, S, dense, err);
  d.det = (p->flags & SANTA_DETERMINISTIC) ? 1 : 0;
  const size_t ns_min = ((size_t)p->max_n_k + santa::kMinSplit - 1) / santa::kMinSplit;
  d.slot_words = santa::slot_words_for((size_t)p->batch * p->num_kv_heads * ns_min * d.G);  // as layout_of
  return d;
}

// Launch shape.  Dense: grid = all items if they fit the resident capacity,
// else the capacity (splits of kMinSplit keys for small problems).  Sampling
// kernel:
//  - the plain fp16 cache, when splits of kSplit keys would leave CUs idle
//    (fewer items than CUs) and splits of kMinSplit keys fit two workgroups
//    per CU: splits of kMinSplit keys, one per workgroup (variant 3; at the
//    Llama layer, B=1, where kSplit items exactly fill the CUs, the shorter
//    splits measured 19.9 us against 17.0: twice the output atomics per row);
//  - else, when every kSplit item fits one workgroup per CU: one item per
//    workgroup (variant 1);
//  - else two workgroups per CU take the items in turn (variant 2); a group's
//    splits must then fit in the grid, for the cross-workgroup waits.
int choose_grid(DecodeParams& d, int kind) {
  d.occ = 1;
  d.split = santa::kSplit;
  const long long groups = (long long)d.B * d.Hkv;
  auto set_split = [&](int split) {
    d.split = split;
    d.ns = (d.max_n_k + split - 1) / split;
    d.total_items = (int)(groups * d.ns);
  };
  set_split(santa::kSplit);
  int cap = capacity(d.D, d.G, kind, 1);
  if (cap <= 0) return SANTA_ERR_HIP;
  if (kind == santa::kOpDense) {
    // splits of kMinSplit keys when kSplit items would leave CUs idle and the
    // shorter ones fit at once (context sweep, B=4 at 4096 keys: 21.8 us
    // against 26.7; not at the Llama layer, B=1, where kSplit items fill the
    // CUs: 36.2 us against 31.3)
    const long long items = groups * ((d.max_n_k + santa::kMinSplit - 1) / santa::kMinSplit);
    if (d.total_items < cu_count() && items <= cap) set_split(santa::kMinSplit);
    d.grid = d.total_items < cap ? d.total_items : cap;
    // every item resident at once: the splits of a group merge each other's
    // records (no last-arrival merge)
    d.exch = d.grid == d.total_items && d.ns <= santa::kMaxExchSplits ? 1 : 0;
    return SANTA_OK;
  }
  if (kind == santa::kOpDecode && d.total_items < cu_count()) {
    const int cap3 = capacity(d.D, d.G, kind, 3, santa::kMinSplit);
    const long long items = groups * ((d.max_n_k + santa::kMinSplit - 1) / santa::kMinSplit);
    if (cap3 > 0 && items <= cap3) {
      set_split(santa::kMinSplit);
      d.occ = 3;
      d.grid = d.total_items;
      return SANTA_OK;
    }
  }
  if (d.total_items > cap) {
    d.occ = 2;
    cap = capacity(d.D, d.G, kind, 2);
    if (cap <= 0) return SANTA_ERR_HIP;
  }
  d.grid = d.total_items < cap ? d.total_items : cap;
  if (d.grid < d.total_items && d.ns > d.grid) return SANTA_ERR_UNSUPPORTED;
  return SANTA_OK;
}

int sampled_step(const santa_problem* p, const void* q, const void* K, const void* V, const int32_t* n_k,
                 int32_t S, int32_t mode, uint64_t seed, float* out, int32_t* indices_out, float* scores_out,
                 uint8_t* kept_out, const float* k_scale, const Paging& pg, void* ws, size_t ws_bytes, void* stream,
                 int kind, int budget = 0, uint32_t* err = nullptr) {
  if (S < 1 || S > SANTA_MAX_S) return p && q && K && V && n_k && out ? SANTA_ERR_SHAPE : SANTA_ERR_NULL;
  int st = common_checks(p, q, K, V, n_k, out, ws, ws_bytes, false, S);
  if (st != SANTA_OK) return st;
  if (kind == santa::kOpDecodeF8) {
    if (!k_scale) return SANTA_ERR_NULL;
    if (!aligned(k_scale, 4)) return SANTA_ERR_ALIGN;
    if (group_size(p) > p->head_dim / 16) return SANTA_ERR_UNSUPPORTED;  // d = 64 with G = 8
  }
  if (mode != SANTA_IID && mode != SANTA_STRATIFIED && mode != SANTA_SYSTEMATIC && mode != SANTA_GUMBEL)
    return SANTA_ERR_MODE;
  if (mode == SANTA_GUMBEL && kind != santa::kOpDecode) return SANTA_ERR_UNSUPPORTED;
  if ((indices_out && !aligned(indices_out, 4)) || (scores_out && !aligned(scores_out, 4))) return SANTA_ERR_ALIGN;
  const bool bern = kind == santa::kOpBernoulli || kind == santa::kOpBernoulliBudget;
  if (bern && p->max_n_k % santa::kTile != 0) return SANTA_ERR_SHAPE;
  if (kind == santa::kOpBernoulliBudget && (budget < 1 || budget > p->head_dim)) return SANTA_ERR_SHAPE;
  DecodeParams d = base_params(p, q, K, V, n_k, out, ws, ws_bytes, S, false, err);
  d.idx_out = indices_out;
  d.scores_out = scores_out;
  d.kept_out = kept_out;
  d.k_scale = k_scale;
  d.block_table = pg.block_table;
  d.lg_block = pg.lg_block;
  d.num_blocks = pg.num_blocks;
  d.budget = budget;
  d.S = S;
  d.mode = mode;
  d.seed = seed;
  if (mode == SANTA_GUMBEL) {
    // no cross-workgroup wait: any grid; four workgroups per CU at most
    const int cus = cu_count();
    if (cus <= 0) return SANTA_ERR_HIP;
    d.grid = d.total_items < 4 * cus ? d.total_items : 4 * cus;
    const hipError_t e = santa::launch_gumbel(d, (hipStream_t)stream);
    return e == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
  }
  st = choose_grid(d, kind);
  if (st != SANTA_OK) return st;
  if (bern) {
    // every group's ternary (or budget) query, drawn once per call
    const hipError_t e = santa::launch_bernoulli_prep(d, key_kind(kind), (hipStream_t)stream);
    if (e != hipSuccess) return SANTA_ERR_HIP;
  }
  const hipError_t e = santa::launch_decode(d, key_kind(kind), (hipStream_t)stream);
  return e == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

}  // namespace

namespace santa {
// santa_decode on a workspace the library owns (the allocation-free entry
// point): error bits go to `err` when it is not null.
int decode_on(const santa_problem* problem, const void* q, const void* K, const void* V, const int32_t* n_k,
              int32_t S, int32_t mode, uint64_t seed, float* out, int32_t* indices_out, float* scores_out,
              void* workspace, size_t workspace_bytes, uint32_t* err, void* stream) {
  if (err && !aligned(err, 4)) return SANTA_ERR_ALIGN;
  return sampled_step(problem, q, K, V, n_k, S, mode, seed, out, indices_out, scores_out, nullptr, nullptr,
                      Paging{}, workspace, workspace_bytes, stream, kOpDecode, 0, err);
}
// Bytes a sampling call needs in a fixed-size buffer shared by problems of
// any size: its tagged part and its untagged part must each fit in half of the
// data area, so that no call's tagged words overlap another's untagged data.
size_t sampling_workspace_bytes(const santa_problem* problem, int32_t S) {
  if (!problem_ok(problem) || S < 1 || S > SANTA_MAX_S) return 0;
  const Layout L = layout_of(problem, S);
  const size_t u = L.acc + L.win + L.bern, half = L.stats > u ? L.stats : u;
  return kHeaderBytes + kCounterBytes + 2 * half;
}
}  // namespace santa

extern "C" {

size_t santa_workspace_bytes(const santa_problem* problem, int32_t S) {
  if (!problem_ok(problem) || S < 1 || S > SANTA_MAX_S) return 0;
  return layout_of(problem, S).total();
}

int santa_decode(const santa_problem* problem, const void* q, const void* K, const void* V, const int32_t* n_k,
                 int32_t S, int32_t mode, uint64_t seed, float* out, int32_t* indices_out, float* scores_out,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return sampled_step(problem, q, K, V, n_k, S, mode, seed, out, indices_out, scores_out, nullptr, nullptr, Paging{},
                      workspace, workspace_bytes, stream, santa::kOpDecode);
}

int santa_decode_paged(const santa_problem* problem, const void* q, const void* K_cache, const void* V_cache,
                       const int32_t* block_table, int32_t block_size, int32_t num_blocks, const int32_t* n_k,
                       int32_t S, int32_t mode, uint64_t seed, float* out, int32_t* indices_out,
                       float* scores_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!problem) return SANTA_ERR_NULL;
  if (!block_table) return SANTA_ERR_NULL;
  if (!aligned(block_table, 4)) return SANTA_ERR_ALIGN;
  int lg = 0;
  while (lg < 11 && (1 << lg) < block_size) ++lg;
  if (block_size < 16 || block_size > santa::kSplit || (1 << lg) != block_size) return SANTA_ERR_SHAPE;
  if (problem->max_n_k % block_size != 0 || num_blocks < 1) return SANTA_ERR_SHAPE;
  Paging pg;
  pg.block_table = block_table;
  pg.lg_block = lg;
  pg.num_blocks = num_blocks;
  return sampled_step(problem, q, K_cache, V_cache, n_k, S, mode, seed, out, indices_out, scores_out, nullptr,
                      nullptr, pg, workspace, workspace_bytes, stream, santa::kOpDecodePaged);
}

int santa_decode_fp8k(const santa_problem* problem, const void* q, const void* K8, const float* k_scale,
                      const void* V, const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, float* out,
                      int32_t* indices_out, float* scores_out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return sampled_step(problem, q, K8, V, n_k, S, mode, seed, out, indices_out, scores_out, nullptr, k_scale,
                      Paging{}, workspace, workspace_bytes, stream, santa::kOpDecodeF8);
}

int santa_bernoulli_qk(const santa_problem* problem, const void* q, const void* K_fm, const void* V,
                       const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, float* out,
                       int32_t* indices_out, float* scores_out, uint8_t* kept_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return sampled_step(problem, q, K_fm, V, n_k, S, mode, seed, out, indices_out, scores_out, kept_out, nullptr,
                      Paging{}, workspace, workspace_bytes, stream, santa::kOpBernoulli);
}

int santa_bernoulli_qk_budget(const santa_problem* problem, const void* q, const void* K_fm, const void* V,
                              const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, int32_t budget,
                              float* out, int32_t* indices_out, float* scores_out, uint8_t* kept_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return sampled_step(problem, q, K_fm, V, n_k, S, mode, seed, out, indices_out, scores_out, kept_out, nullptr,
                      Paging{}, workspace, workspace_bytes, stream, santa::kOpBernoulliBudget, budget);
}

int santa_dense_decode(const santa_problem* problem, const void* q, const void* K, const void* V,
                       const int32_t* n_k, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = common_checks(problem, q, K, V, n_k, out, workspace, workspace_bytes, true);
  if (st != SANTA_OK) return st;
  if ((long long)problem->batch * problem->num_kv_heads > santa::kMaxDenseGroups) return SANTA_ERR_UNSUPPORTED;
  DecodeParams d = base_params(problem, q, K, V, n_k, out, workspace, workspace_bytes, 1, true);
  st = choose_grid(d, santa::kOpDense);
  if (st != SANTA_OK) return st;
  const hipError_t e = santa::launch_dense(d, (hipStream_t)stream);
  return e == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

int santa_pack_k_feature_major(const santa_problem* problem, const void* K, void* K_fm, void* stream) {
  if (!problem || !K || !K_fm) return SANTA_ERR_NULL;
  if (!problem_ok(problem)) return SANTA_ERR_SHAPE;
  if (!supported(problem)) return SANTA_ERR_UNSUPPORTED;
  if (problem->max_n_k % santa::kTile != 0) return SANTA_ERR_SHAPE;
  if (!aligned(K, 16) || !aligned(K_fm, 16)) return SANTA_ERR_ALIGN;
  const hipError_t e = santa::launch_pack_feature_major(K, K_fm, problem->batch, problem->num_kv_heads,
                                                        problem->max_n_k, problem->head_dim, (hipStream_t)stream);
  return e == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

int santa_stream_read(const void* buf, size_t bytes, int32_t workgroups_per_cu, uint32_t* sink, void* stream) {
  if (!buf || !sink) return SANTA_ERR_NULL;
  if (bytes % 16 != 0 || workgroups_per_cu < 1 || workgroups_per_cu > 8) return SANTA_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return SANTA_ERR_ALIGN;
  const hipError_t e = santa::launch_stream_read(buf, bytes, workgroups_per_cu, sink, (hipStream_t)stream);
  return e == hipSuccess ? SANTA_OK : SANTA_ERR_HIP;
}

int santa_workspace_error(const void* workspace, uint32_t* flags, void* stream) {
  if (!workspace || !flags) return SANTA_ERR_NULL;
  if (hipMemcpyAsync(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess)
    return SANTA_ERR_HIP;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SANTA_ERR_HIP;
  return SANTA_OK;
}

const char* santa_status_string(int status) {
  switch (status) {
    case SANTA_OK: return "SANTA_OK";
    case SANTA_ERR_NULL: return "SANTA_ERR_NULL: a required pointer is NULL";
    case SANTA_ERR_SHAPE: return "SANTA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case SANTA_ERR_UNSUPPORTED: return "SANTA_ERR_UNSUPPORTED: head_dim, group size or cache length not supported";
    case SANTA_ERR_ALIGN: return "SANTA_ERR_ALIGN: misaligned pointer";
    case SANTA_ERR_WORKSPACE: return "SANTA_ERR_WORKSPACE: workspace missing or too small";
    case SANTA_ERR_HIP: return "SANTA_ERR_HIP: HIP runtime or launch failure";
    case SANTA_ERR_MODE: return "SANTA_ERR_MODE: unknown sampling mode";
    default: return "unknown santa status";
  }
}

int32_t santa_abi_version(void) { return SANTA_ABI_VERSION; }

}  // extern "C"
