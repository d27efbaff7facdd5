/*
 * libsanta: SANTA stochastic sparse decode-step attention on MI355X (gfx950).
 *
 * The operations follow the abstract of "Stochastic Sparse Attention for
 * Memory-Bound Inference" (arXiv 2605.01910):
 *
 *   - santa_decode: score every key of the KV cache, form the post-softmax
 *     distribution, draw S key indices from it (i.i.d., stratified, or
 *     systematic with one offset), gather only those S value rows and average
 *     them.  This is the abstract's SANTA estimator (its second and third
 *     sentences: a few key indices drawn from the softmax weights, their value
 *     rows added and averaged, which estimates the softmax-weighted value sum
 *     without bias) with the variance-reduced stratified and systematic
 *     variants of its fourth sentence.
 *   - santa_dense_decode: the exact softmax(scale q K^T) V, reading all of K
 *     and V, split over the key sequence (FlashDecoding style; the baseline
 *     the abstract compares against).
 *   - santa_decode_fp8k: santa_decode on a key cache stored as 8-bit floats
 *     (OCP E4M3) with one scale per (sequence, KV head).
 *   - santa_decode_paged: santa_decode on a paged KV cache (block table).
 *   - santa_bernoulli_qk: the abstract's Bernoulli qK^T sampling, which
 *     replaces each query by a stochastic ternary vector so that only the kept
 *     key features are read in the score stage, followed by the SANTA value
 *     stage.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Shapes: B sequences, H_q query heads, H_kv KV heads (G = H_q / H_kv query
 *  heads share a KV head: query head h reads KV head h / G), head dimension d.
 *  Layouts (all row-major, fp16 = IEEE binary16):
 *    q        [B][H_q][d]              fp16
 *    K, V     [B][H_kv][max_n_k][d]    fp16; sequence b uses rows 0..n_k[b]-1
 *    K_fm     [B][H_kv][max_n_k/64][d][64] fp16 (Bernoulli only; see
 *             santa_pack_k_feature_major)
 *    n_k      [B]                      int32, in device memory
 *    out      [B][H_q][d]              fp32
 *    indices  [B][H_q][S]              int32, ascending key indices (optional)
 *    scores   [B][H_q][max_n_k]        fp32 scale * <q, k_j> (optional, debug)
 *  Every pointer argument except `problem` is a device pointer.
 *  Score: s_j = scale * <q, k_j>; the softmax is taken over j < n_k[b].
 *
 *  Ownership: the caller owns every buffer.  The library allocates no device
 *  memory, keeps no pointer after a call returns, and never synchronises:
 *  kernels are enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *  the caller keeps all buffers alive until the stream has completed them.
 *
 *  Workspace: a 256-byte aligned device buffer of at least
 *  santa_workspace_bytes(problem, S) bytes, zero-filled by the caller once
 *  before first use.  The first 1 KiB holds the error bits and counters, and
 *  a 64 KiB region of the dense kernel's arrival counters follows.  The data
 *  of a call comes in two parts:
 *   - words tagged with a launch number: the sampling kernel's per-split
 *     statistics slots, or the dense kernel's records when its splits
 *     exchange them (every work item resident at once).  They grow from the
 *     start of the data area;
 *   - untagged data, placed at the end of the buffer as passed: the exact
 *     sums, Gumbel-max winners, prepared Bernoulli queries, or the dense
 *     kernel's float records.  Each call writes (or clears) this data before
 *     reading it.
 *  The launch number comes from the launch counters, which every tagged call
 *  advances; a tagged word is accepted only with the current number.  The
 *  dense kernel's work counter and arrival counters must be zero when a call
 *  starts, and every call leaves them at zero; the launch counters only grow.
 *  No data region overlaps the header or the arrival counters.
 *  santa_workspace_bytes(P, S) leaves room for the larger tagged part and the
 *  larger untagged part of P's calls of every kind.  So a buffer of that size
 *  serves any sequence of calls, of any entry point, whose problems are no
 *  larger than P in any dimension and whose S is at most S.  This includes
 *  replays of a captured HIP graph.  Every call must pass the same
 *  workspace_bytes; the tagged words of one call then never overlap the
 *  untagged data of another.  Calls that share one workspace must not
 *  run concurrently.  After a call that reported a device error
 *  (santa_workspace_error != 0) the workspace must be zero-filled again.
 *
 *  Waits between workgroups: a sampling call, and santa_dense_decode when
 *  every work item has its own resident workgroup, has workgroups of one
 *  launch wait for statistics that other workgroups of that launch publish.
 *  The grid is sized to what the device keeps resident, so the waits end
 *  when the launch has the device to itself; one that shares it with other
 *  work waits until that work leaves room.  Every wait is bounded: after
 *  about 2^20 polling rounds a workgroup sets bit 0 of the workspace error
 *  bits and goes on, so no call hangs, and its results are then invalid.
 *
 *  Errors: every entry point returns a santa_status.  Arguments are checked
 *  on the host before any HIP call; on a check failure nothing is enqueued.
 *  n_k lives in device memory and cannot be checked without a sync: a
 *  sequence with n_k[b] < 1 or n_k[b] > max_n_k yields NaN outputs (and index
 *  -1) for all its heads.  Asynchronous device faults surface at the caller's
 *  next synchronisation.
 *
 *  Randomness: `seed` (64 bits) is the whole random state of a call.  The
 *  uniforms come from the counter-based generator Philox4x32-10 (Salmon et
 *  al., SC'11): uniform k of stream (row, tag) is output word (k & 3) of
 *  Philox4x32-10 on counter (k >> 2, row, tag, 0) with key (seed low 32 bits,
 *  seed high 32 bits), mapped to (word >> 8) * 2^-24.  row = b * H_q + h for
 *  value sampling; tags are the ASCII codes 'SYST' (systematic offset),
 *  'STRT' (stratified), 'IID ' (i.i.d.), 'BERN' (Bernoulli features, row
 *  b * H_kv + h_kv), 'GUMB' (Gumbel-max draws; see SANTA_GUMBEL).  Equal
 *  inputs and seed give bit-identical sampled indices.  Outputs of the
 *  sampling calls are bit-reproducible with the SANTA_DETERMINISTIC flag (and
 *  always in the SANTA_GUMBEL mode); without it the splits of the key
 *  sequence add their fp32 shares into `out` atomically in whatever order
 *  they finish, so outputs may differ between runs in the last bits.
 *  santa_dense_decode merges its splits in a fixed order and is
 *  bit-reproducible.
 */
#ifndef SANTA_H_
#define SANTA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum santa_status {
  SANTA_OK = 0,
  SANTA_ERR_NULL = 1,        /* a required pointer is NULL */
  SANTA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes, S, scale */
  SANTA_ERR_UNSUPPORTED = 3, /* head_dim, group size or n_k range not built */
  SANTA_ERR_ALIGN = 4,       /* q/K/V/K_fm not 16-byte or out/indices/scores/n_k not 4-byte aligned */
  SANTA_ERR_WORKSPACE = 5,   /* workspace NULL, not 256-byte aligned, or smaller than santa_workspace_bytes */
  SANTA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed */
  SANTA_ERR_MODE = 7         /* unknown sampling mode */
} santa_status;

/* Sampling schemes for the S points t_0 <= ... <= t_{S-1} in [0, 1):
 *  SANTA_IID:        S independent uniforms, sorted;
 *  SANTA_STRATIFIED: t_k = (k + u_k) / S, one uniform per stratum;
 *  SANTA_SYSTEMATIC: t_k = (k + u) / S, one uniform offset for all strata.
 * Point t selects the key j with F_{j-1} <= t < F_j, F the CDF of the
 * post-softmax distribution in key order (F_{-1} = 0).
 *  SANTA_GUMBEL:     S i.i.d. draws by the Gumbel-max trick instead of the
 *                    inverse CDF (santa_decode only): draw k selects
 *                    argmax_j (s_j - log(-log u_kj)), u_kj = ((x >> 9) + 1/2)
 *                    * 2^-23 with x = word (j & 3) of Philox4x32-10 at counter
 *                    (j >> 2, row, 'GUMB', k); the smaller key on a tie; the
 *                    indices are returned ascending and `out` is the exact sum
 *                    of the rows rounded once (bit-reproducible).  It costs
 *                    S * n_k generator words and logarithms per query head. */
typedef enum santa_mode { SANTA_IID = 0, SANTA_STRATIFIED = 1, SANTA_SYSTEMATIC = 2, SANTA_GUMBEL = 3 } santa_mode;

/* Problem description (host memory, read during the call only). */
typedef struct santa_problem {
  int32_t batch;        /* B >= 1 */
  int32_t num_q_heads;  /* H_q >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads; /* H_kv >= 1; G = H_q / H_kv must be 1, 2, 4 or 8 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t max_n_k;      /* rows reserved per (sequence, KV head) in K and V, >= 1 */
  float scale;          /* finite; score = scale * <q, k> (typically 1/sqrt(d)) */
  uint32_t flags;       /* 0 or SANTA_DETERMINISTIC; other bits are rejected (SANTA_ERR_UNSUPPORTED) */
} santa_problem;

/* santa_problem.flags bit of the sampling entry points: `out` is computed as
 * the exact sum of the gathered value rows (times their counts), rounded once
 * to fp32 after the division by S, so equal inputs and seed give bit-identical
 * outputs on every run.  Without it the splits of the key sequence add their
 * fp32 shares atomically in the order they finish (faster: no wait for the
 * last share), and outputs may differ between runs in the last bits.
 * santa_dense_decode ignores the flag: it always merges in a fixed order. */
#define SANTA_DETERMINISTIC 1u

/* Largest sample count accepted by santa_decode / santa_bernoulli_qk. */
#define SANTA_MAX_S 1024

/* Bytes of device workspace that every entry point needs for `problem` and
 * sample count S (1 .. SANTA_MAX_S; 0 if the problem or S is invalid).  A
 * buffer of this size serves calls with any S' <= S. */
size_t santa_workspace_bytes(const santa_problem* problem, int32_t S);

/* SANTA decode step (the abstract's estimator, its second to fourth sentences).
 *   out[b][h] = (1/S) * sum_k V[b][h/G][i_k],  i_k drawn by `mode` from the
 *   post-softmax distribution of scale * q[b][h] . K[b][h/G][j], j < n_k[b].
 * S in [1, SANTA_MAX_S] (S may exceed n_k: sampling is with replacement).
 * indices_out (nullable): the S sampled key indices per head, ascending.
 * scores_out (nullable, debug): the fp32 scores the sampler used.
 * When the problem has more splits of 1024 keys than the device keeps
 * resident workgroups, ceil(max_n_k / 1024) may not exceed that resident
 * count (at least 256 on MI355X, so max_n_k <= 262144 is always accepted);
 * larger caches return SANTA_ERR_UNSUPPORTED. */
int santa_decode(const santa_problem* problem, const void* q, const void* K, const void* V,
                 const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, float* out,
                 int32_t* indices_out, float* scores_out, void* workspace, size_t workspace_bytes,
                 void* stream);

/* SANTA decode step on an fp8 key cache (the same estimator as santa_decode;
 * the abstract calls SANTA complementary to quantization, and keys are almost
 * all of its bytes).
 *   K8      [B][H_kv][max_n_k][d] bytes, each an OCP 8-bit floating point
 *           number in the E4M3 encoding (sign, 4 exponent bits with bias 7, 3
 *           mantissa bits; S.1111.111 is NaN; largest finite magnitude 448)
 *   k_scale [B][H_kv] fp32, device memory: the cache holds
 *           K[b][h][j][i] = k_scale[b][h] * E4M3(K8[b][h][j][i])
 * Scores are scale * k_scale[b][h/G] * <q, decoded K8 row>, the E4M3 values
 * converted exactly to fp16 and accumulated in fp32.  V stays fp16 and every
 * other argument, output and error is as for santa_decode.  d = 64 supports
 * G <= 4 (SANTA_ERR_UNSUPPORTED for G = 8); k_scale must be 4-byte aligned and
 * K8 16-byte aligned. */
int santa_decode_fp8k(const santa_problem* problem, const void* q, const void* K8, const float* k_scale,
                      const void* V, const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, float* out,
                      int32_t* indices_out, float* scores_out, void* workspace, size_t workspace_bytes,
                      void* stream);

/* SANTA decode step on a paged KV cache (the batched serving setting the
 * pages evaluate in, without padding every sequence to max_n_k).
 *   K_cache, V_cache [num_blocks][H_kv][block_size][d] fp16: a pool of
 *            blocks; block p holds block_size consecutive keys (values) of
 *            one sequence, for every KV head
 *   block_table [B][max_n_k / block_size] int32, device memory: key j of
 *            sequence b is row j % block_size of block
 *            block_table[b][j / block_size] (entries past ceil(n_k[b] /
 *            block_size) are not read)
 * block_size: a power of two in [16, 1024] dividing problem->max_n_k (the
 * longest sequence the table can describe).  Every other argument, output and
 * error is as for santa_decode.  A block-table entry outside [0, num_blocks)
 * is read as block 0 and sets bit 1 of the workspace error bits
 * (santa_workspace_error); the results of that sequence are then unspecified. */
int santa_decode_paged(const santa_problem* problem, const void* q, const void* K_cache, const void* V_cache,
                       const int32_t* block_table, int32_t block_size, int32_t num_blocks, const int32_t* n_k,
                       int32_t S, int32_t mode, uint64_t seed, float* out, int32_t* indices_out,
                       float* scores_out, void* workspace, size_t workspace_bytes, void* stream);

/* Exact decode attention: out[b][h] = softmax(scale q K^T) V over j < n_k[b]
 * (the FlashDecoding-style baseline named in the abstract's fifth sentence). */
int santa_dense_decode(const santa_problem* problem, const void* q, const void* K, const void* V,
                       const int32_t* n_k, float* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Bernoulli qK^T step (the abstract's stochastic ternary queries) followed by
 * the SANTA value stage.  For KV head (b, h_kv) one uniform u_i per feature i
 * (stream 'BERN', row b * H_kv + h_kv) is shared by its G query heads; head h
 * keeps feature i iff u_i * A_h < |q_hi| with A_h = max_i |q_hi|, and the kept
 * feature's query value becomes sign(q_hi) * A_h (so E[q~] = q).  Scores use
 * q~ and read only the union of the group's kept features from K_fm.
 * K_fm: feature-major K (max_n_k must be a multiple of 64).  V: row-major.
 * kept_out (nullable): [B][H_q][d] uint8 mask of kept features. */
int santa_bernoulli_qk(const santa_problem* problem, const void* q, const void* K_fm, const void* V,
                       const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, float* out,
                       int32_t* indices_out, float* scores_out, uint8_t* kept_out, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Budget variant of santa_bernoulli_qk: head h keeps feature i with
 * probability pi_i = min(1, budget * |q_hi| / ||q_h||_1) (decided exactly on
 * the group-shared uniform u_i, same stream as santa_bernoulli_qk), so about
 * `budget` features per head are kept, and a kept feature takes the value
 * q_hi / pi_i: q_hi itself where pi_i = 1, sign(q_hi) * ||q_h||_1 / budget
 * otherwise (E[q~] = q).  budget: 1 .. d.  Everything else is as for
 * santa_bernoulli_qk. */
int santa_bernoulli_qk_budget(const santa_problem* problem, const void* q, const void* K_fm, const void* V,
                              const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, int32_t budget,
                              float* out, int32_t* indices_out, float* scores_out, uint8_t* kept_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Relayout a row-major K [B][H_kv][max_n_k][d] into the 64-key feature-major
 * tiles read by santa_bernoulli_qk: K_fm[b][h][t][i][x] = K[b][h][64 t + x][i].
 * max_n_k must be a multiple of 64; K and K_fm must not overlap. */
int santa_pack_k_feature_major(const santa_problem* problem, const void* K, void* K_fm, void* stream);

/* Allocation-free santa_decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments and results as santa_decode, with
 * the workspace in device memory that the library owns instead of a caller's
 * buffer.  Each GPU the library runs on holds one array of
 * SANTA_NOALLOC_SCRATCH_BYTES bytes for the rest of the process.  Its data area
 * past the 65 KiB of header and counters is split in two halves, one for the
 * tagged part of every call and one for the untagged part, so that calls of
 * any size can follow each other.  A problem whose statistics slots or whose
 * other data would exceed a half returns SANTA_ERR_WORKSPACE.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first call
 * on a device takes the array's device address and enqueues a one-word clear
 * on `stream`.  All calls on one GPU share its array: calls that overlap on one
 * GPU (concurrent streams, threads) race and must be serialised by the caller.
 * error_flags (nullable, device memory, 4 bytes): receives, OR-ed in, the
 * device error bits of santa_workspace_error (the caller clears it); without
 * it, device errors of this path are not reported. */
#define SANTA_NOALLOC_SCRATCH_BYTES (16u << 20)
int santa_decode_noalloc(const santa_problem* problem, const void* q, const void* K, const void* V,
                         const int32_t* n_k, int32_t S, int32_t mode, uint64_t seed, float* out,
                         int32_t* indices_out, float* scores_out, uint32_t* error_flags, void* stream);

/* Measurement utility (not part of the decode step): read `bytes` bytes of the
 * device buffer `buf` once with the 16-byte non-temporal loads the decode
 * kernels stream K with, using workgroups_per_cu (1..8) workgroups of 256
 * threads per compute unit, each reading one contiguous range with two
 * buffers of 16, 8 or 4 loads per lane in flight (1, 2, or more workgroups
 * per CU: the same bytes in flight per CU).  Nothing is
 * written except, practically never, one word of `sink` (device memory, 4
 * bytes): the loaded words are folded into a value that is stored only if it
 * equals a fixed constant, so the loads cannot be optimised away.  It gives
 * the bandwidth a bare read of the decode step's bytes reaches in one launch.
 * bytes must be a multiple of 16 and buf 16-byte aligned. */
int santa_stream_read(const void* buf, size_t bytes, int32_t workgroups_per_cu, uint32_t* sink, void* stream);

/* Copy the device error bits of a workspace to *flags (synchronises `stream`).
 * Bit 0: a bounded cross-workgroup wait timed out (results invalid).
 * Bit 1: a block-table entry of santa_decode_paged was out of range. */
int santa_workspace_error(const void* workspace, uint32_t* flags, void* stream);

/* Human-readable name of a status code (static string). */
const char* santa_status_string(int status);

/* ABI version of this header (incremented on incompatible changes). */
#define SANTA_ABI_VERSION 3
int32_t santa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SANTA_H_ */
