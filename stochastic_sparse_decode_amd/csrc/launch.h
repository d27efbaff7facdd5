// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace santa {

constexpr int kThreads = 256;   // threads per workgroup (4 waves)
constexpr int kWaves = kThreads / 64;
constexpr int kSplit = 1024;    // keys per work item (one split of one KV head)
constexpr int kMinSplit = 512;  // shorter splits of the plain fp16 cache (small problems)
constexpr int kMaxS = 1024;     // largest sample count
constexpr int kTile = 64;       // keys per feature-major tile (Bernoulli mode)
constexpr uint32_t kSpinLimit = 1u << 20;  // bounded wait: ~1 s, then error flag
constexpr uint64_t kLaunchUnit = 1ull << 20;  // launch counter increment per launch (> any grid)
constexpr int kLaunchCounters = 7;     // the launch count is the sum of 7 counters, one per 128-byte line
constexpr int kLaunchStride = 16;      // uint64 words between the counters
constexpr int kBernRecord = 291;       // 16-byte words of one group's prepared Bernoulli query

// Error bits written by kernels into the workspace header.
constexpr uint32_t kErrSpinTimeout = 1u;
constexpr uint32_t kErrBlockTable = 2u;  // a block-table entry out of range (read as block 0)

// Device pointers carved out of the caller's workspace.  The words that must
// be zero when a launch starts (the dense kernel's work counter and arrival
// counters; every dense launch leaves them at zero) sit in the header and in a
// counter region of fixed size right after it, which no other region of any
// problem ever overlaps; statistics slots carry the launch's tag and partial
// records are written before they are read, so a buffer can serve problems of
// different sizes.
// Dense kernel: splits per group up to which the resident grid merges by
// exchange (each split merges F / ns of the group's G * D features).
constexpr int kMaxExchSplits = 128;
constexpr int kMaxDenseGroups = 16384;  // B * H_kv of a dense step (its counters fill 64 KiB)
struct Workspace {
  uint32_t* err;        // error bits (never cleared by kernels)
  uint32_t* work_ctr;   // dense kernel: dynamic work-item counter, returns to 0 at kernel end
  uint64_t* launches;   // launch counters of the tagged launches, sampling and dense (their sum grows by
                        // kLaunchUnit per launch)
  uint32_t* arrive;     // [groups] dense kernel: splits of the group that stored their record, back to 0
  uint64_t* stats;      // [groups][G][ns][2] (tag:32 | split max bits, tag:32 | split mass bits); sized for
                        // splits of kMinSplit keys
  uint64_t* acc;        // [groups][G][D] exact output sums of the deterministic mode (cleared by split 0 per launch)
  uint64_t* win;        // [B][H_q][S] Gumbel-max draws: (order bits of the value, ~key) winners (cleared per call)
  float* partial;       // [groups][ns][G][D + 2] partial outputs of the dense kernel (acc, m, l)
  uint64_t* xrec;       // the same memory as [groups][ns][G][D + 2] words (tag:32 | value bits): the dense
                        // kernel's records when its splits merge each other's (exch = 1)
  uint4* bern;          // [groups][kBernRecord] Bernoulli step: each group's ternary (or budget) query, prepared once
                        // per call: nu | A[8] | kept-feature list[128] | weights[128] | clipped values[128]
};

// Kernel arguments.  The fields a workgroup needs before its first K load
// (where its split lies, and the query) fill the first 64-byte line, so the
// kernel reads them with one scalar-cache fetch.
struct DecodeParams {
  // ---- first 64 bytes ----
  const void* K;        // [B][Hkv][max_n_k][D] fp16 (row-major) or feature-major tiles
  const int32_t* n_k;   // [B]
  const void* q;        // [B][Hq][D] fp16
  int ns;               // splits per group = ceil(max_n_k / kSplit)
  int max_n_k;
  int Hkv;
  int total_items;      // B * Hkv * ns
  int grid;             // persistent workgroups
  int Hq;
  float scale;
  int S;
  int mode;
  int B;
  // ---- the rest ----
  const void* V;        // [B][Hkv][max_n_k][D] fp16
  float* out;           // [B][Hq][D]
  int32_t* idx_out;     // [B][Hq][S] or null
  float* scores_out;    // [B][Hq][max_n_k] or null
  uint8_t* kept_out;    // [B][Hq][D] or null (Bernoulli)
  const float* k_scale; // [B][Hkv] scales of an fp8 key cache (K = k_scale * decode(K8)), else null
  const int32_t* block_table;  // paged cache: [B][max_n_k / block_size] block of each key range, else null
  int lg_block;         // paged cache: log2(block_size)
  int num_blocks;       // paged cache: blocks in K and V, each [Hkv][block_size][D]
  int budget;           // Bernoulli budget variant: expected kept features per head (m), else 0
  uint64_t seed;
  int D, G;
  int occ;              // sampling kernel variant: 1 = one item per workgroup (one per CU), 2 = items taken in
                        // turn (two workgroups per CU), 3 = one item per workgroup (two per CU)
  int split;            // keys per work item of the sampling kernel: kSplit, or 512 (variant 3, plain fp16 cache)
  int det;              // 1: out is the exact sum of the gathered rows rounded once (bit-reproducible)
  int slot_words;       // 8-byte words per statistics slot: 2, or 16 (one slot per 128-byte line)
  int exch;             // dense kernel: 1 = every item has its own resident workgroup, and the splits of a
                        // group exchange tagged records and each merges a share of the features
  Workspace ws;
};
static_assert(offsetof(DecodeParams, V) == 64, "the fields read first fill one 64-byte line");

// Statistics slots: 16 bytes each, or one per 128-byte line when the padded
// region of a problem stays within kPaddedSlotBytes.  A head's slots are
// polled by every workgroup of its group; with one slot per line, the reads of
// one line come only from the lanes that wait for that slot, and the split
// that writes it shares the line with no other.
constexpr size_t kPaddedSlotBytes = 1u << 20;
inline int slot_words_for(size_t slots) { return slots * 128 <= kPaddedSlotBytes ? 16 : 2; }

enum Op { kOpDecode = 0, kOpDense = 1, kOpBernoulli = 2, kOpDecodeF8 = 3, kOpDecodePaged = 4, kOpBernoulliBudget = 5 };

// Key cache kinds of the sampling kernel.
enum KeyKind { kKeyF16 = 0, kKeyBernoulli = 1, kKeyF8 = 2, kKeyF16Paged = 3, kKeyBernoulliBudget = 4 };
constexpr int kMaxBlocksPerSplit = kSplit / 16;  // smallest block: 16 keys

// Resident-workgroup capacity of the current device for a kernel variant.
int decode_capacity(int D, int G, int key_kind, int variant, int split);
int dense_capacity(int D, int G);

// Bernoulli step: prepares every group's query (one workgroup per group), then the decode kernel.
hipError_t launch_bernoulli_prep(const DecodeParams& p, int key_kind, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int key_kind, hipStream_t stream);
hipError_t launch_dense(const DecodeParams& p, hipStream_t stream);
}  // namespace santa

struct santa_problem;
namespace santa {
int decode_on(const santa_problem* problem, const void* q, const void* K, const void* V, const int32_t* n_k,
              int32_t S, int32_t mode, uint64_t seed, float* out, int32_t* indices_out, float* scores_out,
              void* workspace, size_t workspace_bytes, uint32_t* err, void* stream);
size_t sampling_workspace_bytes(const santa_problem* problem, int32_t S);

hipError_t launch_gumbel(const DecodeParams& p, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups_per_cu, uint32_t* sink,
                              hipStream_t stream);
hipError_t launch_pack_feature_major(const void* K, void* K_fm, int B, int Hkv, int max_n_k, int D,
                                     hipStream_t stream);

}  // namespace santa
