/*
 * ikbo.h -- C ABI of libikbo.so: In-Kernel Broadcast Optimization (IKBO)
 * target attention for MI355X (gfx950).
 *
 * The operation (IKBO blog, "In-Kernel Broadcast Optimization: Co-Designing
 * Kernels for RecSys Inference", sections 1.1-1.3 and 3.1, Fig. 10): a
 * request carries two batch sizes.  Request-only (RO) tensors are per user
 * (here the user's key/value history), non-request-only (NRO) tensors are per
 * candidate (here the candidate queries).  A runtime-supplied mapping names
 * the user of every candidate.  Each candidate query attends, without a causal
 * mask (section 3: the models are encoder-driven), over the whole key/value
 * sequence of its user.  The user sequence is never copied out per candidate:
 * the kernel reads the mapping and indexes the user's K/V itself.  The result
 * equals softmax(scale * q k^T) v computed on an explicitly broadcast K/V.
 *
 * Tensor layouts (row-major, contiguous, element type given by `dtype`):
 *   q_cand   [n_cand, n_q, H, d]   candidate queries (n_q query tokens each)
 *   k_user   [total_len, H, d]     user keys, packed user after user
 *   v_user   [total_len, H, d]     user values, same packing
 *   q_user   [total_len, H, d]     user queries (fused self + target only)
 *   out_cand [n_cand, n_q, H, d]   same dtype as q_cand
 *   out_user [total_len, H, d]     same dtype (fused self + target only)
 *   user_offsets int32 [n_users + 1]: rows of user u are
 *                user_offsets[u] .. user_offsets[u+1]-1; user_offsets[0] = 0.
 *   cand_to_user int32 [n_cand]: user of each candidate, any order.
 * `d` is 32, 64 or 128.  Element types: IKBO_DTYPE_BF16 (bf16 in, fp32
 * accumulation, bf16 out) or IKBO_DTYPE_F32.  Rows must be 16-byte aligned
 * (true for the layouts above with d >= 32 and 16-byte aligned base pointers).
 *
 * Conventions for every entry point:
 *   - Pointers named *_host are host memory; every other tensor pointer is
 *     device memory on the current HIP device.
 *   - `stream` is a hipStream_t (NULL = the default stream); all device work is
 *     enqueued on it, and the call returns before that work completes, except
 *     where a call says it synchronises.
 *   - The caller owns every tensor and must keep it alive until the stream
 *     work completes.  The library owns only its plans and workspaces.
 *   - A plan or handle (plan, LCE, backward, MXFP8) is used by one host thread
 *     at a time; different plans and handles may be used concurrently.  The
 *     entry points without a plan keep one internal plan per (device, stream)
 *     and serialise on it.
 *   - A negative return is an error; nothing has been launched and no output
 *     has been written.  ikbo_last_error() gives a message (thread-local).
 *     No C++ exception crosses this boundary.
 *   - Output rows are fully overwritten.  Results are deterministic: the same
 *     inputs give bitwise-identical outputs, whatever the grid size.
 *   - A user with zero keys but with candidates gets all-zero output rows
 *     (softmax over an empty set is undefined; this library's reading).
 *   - n_cand = 0 is a successful no-op.  n_users = 0 with n_cand > 0 is
 *     IKBO_ERR_BAD_MAPPING.
 */
#ifndef IKBO_H_
#define IKBO_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  IKBO_OK = 0,
  IKBO_ERR_INVALID_ARG = -1, /* null pointer, negative size, H < 1, aliasing output */
  IKBO_ERR_BAD_OFFSETS = -2, /* user_offsets not starting at 0 or decreasing     */
  IKBO_ERR_BAD_MAPPING = -3, /* a cand_to_user entry outside [0, n_users)        */
  IKBO_ERR_UNSUPPORTED = -4, /* d or dtype not supported                          */
  IKBO_ERR_HIP = -5,         /* a HIP runtime call failed                          */
  IKBO_ERR_NOMEM = -6        /* device or pinned host allocation failed            */
};

enum { IKBO_DTYPE_BF16 = 0, IKBO_DTYPE_F32 = 1 };

/* Library version as an integer (major * 10000 + minor * 100 + patch). */
int ikbo_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ikbo_last_error(void);

/*
 * Host-side grouping of candidates by user (CSR).  Host pointers only; no GPU
 * is touched.  The pages hand the kernel the candidate-to-user mapping
 * (IKBO blog section 1.3) and pair neighbouring candidates of one user inside
 * a thread block (section 3.2, Alg. 1); this generalises the pairing to any
 * order and any count.
 *   counts[n_users]          candidates per user
 *   cand_offsets[n_users+1]  exclusive prefix sum of counts
 *   cand_perm[n_cand]        candidate indices sorted by user; ascending
 *                            original index within a user (stable)
 *   tiles[3 * max_tiles]     (u, row_start, row_len) triples: user u owns
 *                            counts[u] * n_q rows, row r being query r % n_q of
 *                            candidate cand_perm[cand_offsets[u] + r / n_q];
 *                            rows are cut into tiles of `bm` (the last may be
 *                            shorter); users ascending, tiles ascending.
 *   *n_tiles                 number of tiles written.
 * Returns IKBO_ERR_INVALID_ARG if max_tiles is too small (then *n_tiles holds
 * the number needed), IKBO_ERR_BAD_MAPPING for an out-of-range mapping.
 */
int ikbo_group_csr(const int32_t* cand_to_user_host, int32_t n_cand, int32_t n_users,
                   int32_t n_q, int32_t bm, int32_t* counts, int32_t* cand_offsets,
                   int32_t* cand_perm, int32_t* tiles, int32_t max_tiles, int32_t* n_tiles);

/*
 * IKBO target attention, bf16, one query token per candidate: the call the
 * problem statement names.  user_offsets and cand_to_user are DEVICE pointers;
 * the call copies them to the host, waits for the stream (one synchronisation),
 * groups candidates on the host, writes the work list to pinned memory that
 * the kernels read in place, and launches.  `scale`
 * multiplies q.k (typically 1/sqrt(d)).  out: [n_cand, 1, H, d] bf16.
 */
int ikbo_attn_fwd(const void* q_cand, const void* k_user, const void* v_user,
                  const int32_t* user_offsets, const int32_t* cand_to_user,
                  int32_t n_users, int32_t n_cand, int32_t H, int32_t d, float scale,
                  void* out, void* stream);

/*
 * As ikbo_attn_fwd with fp32 q, k, v and out (the same arguments; fp32
 * accumulation and exponentials, one query token per candidate).
 */
int ikbo_attn_fwd_f32(const void* q_cand, const void* k_user, const void* v_user,
                      const int32_t* user_offsets, const int32_t* cand_to_user,
                      int32_t n_users, int32_t n_cand, int32_t H, int32_t d, float scale,
                      void* out, void* stream);

/*
 * Multi-target form: as ikbo_attn_fwd, followed by n_q (query tokens per
 * candidate, >= 1) and dtype.  q_cand and out are [n_cand, n_q, H, d]; each
 * query token of a candidate attends on its own over the whole sequence of
 * the candidate's user (IKBO blog section 3.2: several query tokens per
 * candidate).  ikbo_attn_fwd_ex is the same call with n_q and dtype placed
 * next to the other sizes.
 */
int ikbo_attn_fwd_mt(const void* q_cand, const void* k_user, const void* v_user,
                     const int32_t* user_offsets, const int32_t* cand_to_user,
                     int32_t n_users, int32_t n_cand, int32_t H, int32_t d, float scale,
                     void* out, void* stream, int32_t n_q, int32_t dtype);

/*
 * Allocation-free form of ikbo_attn_fwd_mt, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, same planner and kernels; the
 * kernels' scratch (split-KV partials and their row records, the work list and
 * the candidate order) is one fixed library array per device, 64 MiB, held by
 * every device the call runs on until the process ends.  Nothing is allocated
 * per call, on the device or the host: host planning storage is reserved at
 * the first call.  Limits: n_users <= 65536, n_cand <= 1048576, and
 * H * (n_cand * n_q / 128 + n_users + 1) <= 131072 (IKBO_ERR_INVALID_ARG
 * beyond them, before anything is enqueued); when the split partials would
 * not fit, key ranges are left whole (same result within rounding).  The call
 * copies the mapping to the host and waits for the stream, like
 * ikbo_attn_fwd_mt.  All calls on one device share its scratch: calls that
 * overlap in time on one device (other streams, other host threads' streams)
 * race; the library serialises only the host side.
 */
int ikbo_attn_fwd_mt_noalloc(const void* q_cand, const void* k_user, const void* v_user,
                             const int32_t* user_offsets, const int32_t* cand_to_user,
                             int32_t n_users, int32_t n_cand, int32_t H, int32_t d, float scale,
                             void* out, void* stream, int32_t n_q, int32_t dtype);

/* As ikbo_attn_fwd_mt, with n_q and dtype next to the other sizes. */
int ikbo_attn_fwd_ex(const void* q_cand, const void* k_user, const void* v_user,
                     const int32_t* user_offsets, const int32_t* cand_to_user,
                     int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d,
                     float scale, int32_t dtype, void* out, void* stream);

/*
 * Fused self + target attention (IKBO blog section 3.3): both attentions read
 * the same user K/V.  Self rows: query q_user[user_offsets[u] + t] attends
 * causally to keys 0..t of its own user (diagonal included).  Target rows: as
 * ikbo_attn_fwd_ex with n_q = 1 (non-causal over the whole user sequence).
 * One launch covers both kinds of work.
 */
int ikbo_self_target_fwd(const void* q_user, const void* q_cand, const void* k_user,
                         const void* v_user, const int32_t* user_offsets,
                         const int32_t* cand_to_user, int32_t n_users, int32_t n_cand,
                         int32_t H, int32_t d, float scale, int32_t dtype,
                         void* out_user, void* out_cand, void* stream);

/*
 * Materialised-broadcast comparator (measurement only; the broadcast done
 * before dispatch that the IKBO blog section 1.4 and Fig. 10 (left) describe).  A copy kernel first writes a
 * per-candidate copy of its user's K and V into a library-owned buffer
 * [sum_c L_{u(c)}, H, d]; the same attention kernel then runs with the
 * identity mapping.  Arguments as ikbo_attn_fwd_mt; output equals it.  Candidates are processed
 * in chunks so the broadcast buffer stays within IKBO_BCAST_MAX_GB
 * (environment, default 32).  Synchronises like ikbo_attn_fwd.
 */
int ikbo_attn_fwd_materialized(const void* q_cand, const void* k_user, const void* v_user,
                               const int32_t* user_offsets, const int32_t* cand_to_user,
                               int32_t n_users, int32_t n_cand, int32_t H, int32_t d, float scale,
                               void* out, void* stream, int32_t n_q, int32_t dtype);

/*
 * Plans: the host grouping and work list, built from HOST copies of the
 * mapping (as an inference runtime holds them), then reused by launches
 * without any host-device synchronisation.
 *
 * ikbo_plan_create: allocates a plan bound to the current device and builds
 *   it for the request the host mapping describes (as ikbo_plan_build; on
 *   error no plan is returned).
 * ikbo_plan_build: validates, groups candidates (ikbo_group_csr) and builds
 *   the load-balanced work list over (user, head, row tile, key chunk) in a
 *   pinned host buffer that the kernels read in place (no copy is enqueued).
 *   Does not synchronise.  A plan may be rebuilt for a new request at any
 *   time: it uses 16 pinned buffers in turn, and a build waits, if needed,
 *   only for the launches that read its buffer 16 builds earlier (tracked
 *   by an event recorded every 8th launch, not after each one).
 *   with_self = 1 adds causal self-attention rows (then n_q must be 1).
 * ikbo_attn_fwd_planned: launches the attention for the plan's last build.
 *   q_user/out_user are used only when the plan was built with with_self.
 *   Launches of one plan share its split-KV workspace and work-list buffers:
 *   keep them on one stream; a launch on another stream than the plan's
 *   previous one first waits, on the host, for that stream to drain.  Split
 *   groups are merged by a second kernel with the log-sum-exp rule of the
 *   Flash-Decoding split-KV reduction (AI-infra guide, section 4.6.4), in
 *   chunk order, so results do not depend on the schedule or the launch grid.
 * ikbo_attn_fwd_hostmap: ikbo_plan_build followed by ikbo_attn_fwd_planned
 *   in one call (the per-request step of a runtime that holds the mapping on
 *   the host).  The tensors are checked against the new request first; on
 *   any error nothing is launched and the plan keeps its previous build
 *   unless the error came from the build itself.
 * ikbo_attn_fwd_train: ikbo_attn_fwd_planned for a bf16 plan without self
 *   rows that also writes lse [n_cand, n_q, H] (fp32, 4-byte aligned): the
 *   natural-log log-sum-exp of each row's scaled scores over its user's keys,
 *   ln sum_j exp(scale * q . k_j) (-inf for users with no keys), which the
 *   backward takes instead of recomputing it (AI-infra guide, section 4.6.3:
 *   the backward rebuilds P from the scores and the saved statistic).
 *   UNSUPPORTED for fp32 plans and plans with self rows.
 * ikbo_plan_destroy: frees the plan after synchronising its device.
 */
int ikbo_plan_create(const int32_t* user_offsets_host, const int32_t* cand_to_user_host,
                     int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d,
                     int32_t dtype, int32_t with_self, void* stream, void** plan);
int ikbo_plan_build(void* plan, const int32_t* user_offsets_host, const int32_t* cand_to_user_host,
                    int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d,
                    int32_t dtype, int32_t with_self, void* stream);
int ikbo_attn_fwd_planned(void* plan, const void* q_cand, const void* q_user,
                          const void* k_user, const void* v_user, float scale,
                          void* out_cand, void* out_user, void* stream);
int ikbo_attn_fwd_hostmap(void* plan, const int32_t* user_offsets_host, const int32_t* cand_to_user_host,
                          int32_t n_users, int32_t n_cand, int32_t n_q, int32_t H, int32_t d, int32_t dtype,
                          int32_t with_self, const void* q_cand, const void* q_user, const void* k_user,
                          const void* v_user, float scale, void* out_cand, void* out_user, void* stream);
int ikbo_attn_fwd_train(void* plan, const void* q_cand, const void* k_user, const void* v_user, float scale,
                        void* out_cand, float* lse, void* stream);
void ikbo_plan_destroy(void* plan);

/*
 * Kernel timing, for measurement.  ikbo_plan_timing(plan, 1) starts recording
 * HIP events on the launch stream around the attention kernel and around the
 * split-KV merge kernel of each later ikbo_attn_fwd_planned call (at most 4096
 * launches; 0 stops and both calls reset the record).  ikbo_plan_timing_read
 * waits for the recorded events and writes per-launch durations in
 * milliseconds (merge_ms is 0 for launches without split groups); *n receives
 * the number written.
 */
int ikbo_plan_timing(void* plan, int32_t enable);
int ikbo_plan_timing_read(void* plan, float* attn_ms, float* merge_ms, int32_t max_n, int32_t* n);

/*
 * Per-item trace, for load-balance analysis (bf16 kernel).  With tracing on,
 * each later launch of the plan writes one record of 6 int64 per work item, in
 * the plan's item order: [0] logical workgroup << 32 | XCC << 16 | HW_ID
 * CU/SE bits, [1] item start, [2] ring primed and query rows loaded, [3] key
 * loop done, [4] item done (device real-time clock ticks, 100 MHz), [5] key
 * tiles.  ikbo_plan_trace_read synchronises the device and copies the records
 * of the last launch to the host.
 */
int ikbo_plan_trace(void* plan, int32_t enable);
int ikbo_plan_trace_read(void* plan, int64_t* records, int32_t max_items, int32_t* n_items);

/*
 * IKBO linear compression, Type I (IKBO blog section 2: 2.1 the split of the
 * batched projection along K, Fig. 2; 2.2 zero padding of each decomposed K;
 * 2.3 the broadcast-add fused into the candidate GEMM's epilogue, Fig. 3; App. 2
 * gives the shapes B = 1024, M = 433, K = 2044, N = 256).  The linear compression
 * multiplies one learned W [M, K] with every candidate's K input embeddings of
 * width N, (M, K) @ (B, K, N) -> (B, M, N), where a candidate's K embeddings are
 * its user's K_u embeddings followed by its own K_c embeddings.  IKBO computes
 *   y[u]   = W[:, :K_u] . x_user[u]                    once per user (fp32),
 *   out[b] = W[:, K_u:] . x_cand[b] + y[cand_to_user[b]]
 * with fp32 accumulation and bf16 output; the user embeddings are never copied
 * per candidate and the broadcast add happens in registers.
 *
 * ikbo_lce_create: packs W (device, bf16 [M, ldw] row-major, user columns
 *   [0, K_u), candidate columns [K_u, K_u + K_c), ldw >= K_u + K_c) into two
 *   library-owned blocks zero-padded to K multiples of 32 and M multiples of
 *   256 (enqueued on `stream`; W may be freed once that work completes).
 *   M >= 1, K_u >= 0, K_c >= 0, K_u + K_c >= 1.  *lce receives the handle.
 * ikbo_lce_fwd: x_user [n_users, K_u, N], x_cand [n_cand, K_c, N], out
 *   [n_cand, M, N], all bf16 device tensors, 16-byte aligned; cand_to_user is an
 *   int32 device array [n_cand].  N must be a positive multiple of 128.  Enqueues
 *   two kernels (user GEMM, then candidate GEMM) and returns without
 *   synchronising.  Mapping entries outside [0, n_users) are not an error the
 *   call can see: their output rows are written as zeros and counted (see
 *   ikbo_lce_errors).  Calls with one handle must be ordered on one stream (they
 *   share its user-result workspace).  n_cand = 0 is a no-op.
 * ikbo_lce_errors: synchronises the device and returns (and resets) the number
 *   of batch elements (candidates, or vendors and items of a three-level call)
 *   seen with an out-of-range mapping entry since the last call.
 * ikbo_lce_timing / _timing_read: per-call durations of the user and candidate
 *   GEMMs from events stamped by the dispatches (measurement; as the plan
 *   timing functions, at most 4096 calls between resets).
 * ikbo_lce_destroy: frees the handle after synchronising its device.
 */
int ikbo_lce_create(void** lce, const void* w, int32_t M, int32_t K_u, int32_t K_c, int32_t ldw, void* stream);
/*
 * Three levels, user -> ads vendor -> ads item (IKBO blog, conclusion: a user
 * sees several vendors, each vendor offers several items; two nested broadcast
 * relations with independent, uneven ratios).  An item's K embeddings are its
 * user's K_u, its vendor's K_v and its own K_c embeddings; the product nests
 * the Type I split:
 *   y_user[u]   = W[:, :K_u] . x_user[u]                                    (fp32)
 *   y_vendor[v] = W[:, K_u:K_u+K_v] . x_vendor[v] + y_user[vendor_to_user[v]]   (fp32)
 *   out[b]      = W[:, K_u+K_v:] . x_cand[b] + y_vendor[cand_to_vendor[b]]      (bf16)
 * each level at its own batch size, each parent result added in the child
 * GEMM's epilogue; neither broadcast copy is ever written.
 * ikbo_lce3_create: as ikbo_lce_create, W columns user, vendor, item (ldw >=
 *   K_u + K_v + K_c; any block may be empty, the total may not).
 * ikbo_lce3_fwd: x_user [n_users, K_u, N], x_vendor [n_vendors, K_v, N],
 *   x_cand [n_cand, K_c, N], out [n_cand, M, N] (bf16 device tensors, 16-byte
 *   aligned); vendor_to_user [n_vendors] and cand_to_vendor [n_cand] are int32
 *   device arrays.  Four launches (item ordering, user, vendor and item GEMMs),
 *   no synchronisation.  Out-of-range entries give zero results for that vendor
 *   or item and are counted (ikbo_lce_errors).  Timing: the first slot spans the
 *   user and vendor GEMMs, the second the item GEMM.  A handle from
 *   ikbo_lce3_create takes only ikbo_lce3_fwd, one from ikbo_lce_create only
 *   ikbo_lce_fwd (INVALID_ARG otherwise).
 */
int ikbo_lce3_create(void** lce, const void* w, int32_t M, int32_t K_u, int32_t K_v, int32_t K_c, int32_t ldw,
                     void* stream);
int ikbo_lce3_fwd(void* lce, const void* x_user, const void* x_vendor, const void* x_cand,
                  const int32_t* vendor_to_user, const int32_t* cand_to_vendor, int32_t n_users, int32_t n_vendors,
                  int32_t n_cand, int32_t N, void* out, void* stream);
int ikbo_lce_fwd(void* lce, const void* x_user, const void* x_cand, const int32_t* cand_to_user, int32_t n_users,
                 int32_t n_cand, int32_t N, void* out, void* stream);
int ikbo_lce_errors(void* lce, int64_t* count);
int ikbo_lce_timing(void* lce, int32_t enable);
int ikbo_lce_timing_read(void* lce, float* user_ms, float* cand_ms, int32_t max_n, int32_t* n);
void ikbo_lce_destroy(void* lce);

/*
 * Backward of IKBO target attention (IKBO blog section 3.1, Fig. 10 for the
 * forward; section 1.2: the kernels also serve training when candidates
 * outnumber users).  The forward attends each candidate's n_q query rows over
 * its user's K/V without copying it per candidate, so the gradient of a user's
 * K/V is the sum over all its candidates' rows:
 *   dq_cand = scale * dS K,  dk_user = scale * sum dS^T q,  dv_user = sum P^T dO,
 * with P the softmax of scale * q k^T (recomputed from the scores and each
 * row's log-sum-exp, AI-infra guide section 4.6.3), D = rowsum(dout * out) and
 * dS = P * (dout v^T - D).  Two kernels (the guide's two loop orders; the TLX
 * jagged-attention post, section 2.2, for the K/V-block-outer tile list): dQ
 * per row tile and key chunk (plus a merge of split chunks), then dK/dV per
 * 128 keys of a user with the reduction over candidates in registers (no
 * atomics; results are deterministic).
 *
 * ikbo_bwd_create: a handle owning the work lists (pinned host memory, 16
 *   buffers used in turn, as for plans; a call on another stream than the
 *   handle's previous one first waits for that stream) and device workspaces: 4 * (1 + 2H) * (n_cand*n_q +
 *   128) bytes of per-row statistics, and 64 KB + 2 KB per split slot of dQ
 *   partials (long key ranges are split as in the forward and merged in chunk
 *   order, so results stay deterministic).
 * ikbo_attn_bwd: user_offsets [n_users + 1] and cand_to_user [n_cand] are HOST
 *   int32 arrays (as an inference or training runtime holds them); the tensors
 *   are bf16 device arrays, 16-byte aligned, row-major: q_cand, out (the
 *   forward output), dout, dq_cand [n_cand, n_q, H, d]; k_user, v_user,
 *   dk_user, dv_user [user_offsets[n_users], H, d].  d must be 128.  lse is
 *   optional: the forward's log-sum-exp [n_cand, n_q, H] fp32 as
 *   ikbo_attn_fwd_train writes it; given, the dQ kernel takes it instead of
 *   recomputing it (one pass over the keys less), null, it recomputes.  Every
 *   gradient element is written: users with no candidates get zero dk/dv
 *   rows, candidates of users with no keys zero dq rows.  Enqueues two kernels
 *   on `stream` and returns without synchronising (it may wait for the call
 *   before last on the same handle to finish reading its work list).  Errors
 *   (INVALID_ARG: null or misaligned tensors, gradients aliasing inputs or
 *   each other, bad sizes; BAD_OFFSETS; BAD_MAPPING; UNSUPPORTED: d != 128)
 *   launch nothing.  Calls on one handle must be ordered on one stream.
 * ikbo_bwd_info: info[0] dQ work items, info[1] dK/dV work items, info[2] split dQ
 *   groups (key ranges cut into chunks, merged by a third kernel) of the last call.
 * ikbo_bwd_timing / _timing_read: per-call durations of the two kernels from
 *   events stamped by their dispatches (at most 4096 calls between resets).
 * ikbo_bwd_destroy: frees the handle after synchronising its device.
 */
int ikbo_bwd_create(void** bwd);
int ikbo_attn_bwd(void* bwd, const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users,
                  int32_t n_cand, int32_t n_q, int32_t H, int32_t d, float scale, const void* q_cand,
                  const void* k_user, const void* v_user, const void* out, const void* dout, void* dq_cand,
                  void* dk_user, void* dv_user, const float* lse, void* stream);
int ikbo_bwd_info(void* bwd, int64_t* info, int32_t n_info);
int ikbo_bwd_timing(void* bwd, int32_t enable);
int ikbo_bwd_timing_read(void* bwd, float* dq_ms, float* dkv_ms, int32_t max_n, int32_t* n);
void ikbo_bwd_destroy(void* bwd);

/*
 * MXFP8 IKBO target attention (TLX attention post, section 3: the micro-scaled
 * FP8 variant; IKBO blog, section 3.1, Fig. 10 for the broadcast-free target
 * attention it runs).  Inputs are E4M3 codes (OCP FP8: 4 exponent bits, bias
 * 7, 3 mantissa bits, largest finite 448, S.1111.111 NaN) with one E8M0 scale
 * (value 2^(s - 127), 255 NaN) per 32 elements along each product's
 * contraction.  For candidate c of user u, query row r and head h:
 *   x_j = scale * log2(e) * (q^ . k^_j) over the user's keys j, m = an integer
 *   (the result does not depend on which: the kernel lets it lag the running
 *   maximum by up to 8), p_j = 2^(x_j - m);
 *   P^ = p quantized per block of 32 keys (blocks start at the user's first
 *   key): the block's scale is the smallest 2^e with max p <= 448 * 2^e and
 *   each p_j / 2^e is rounded to E4M3 (nearest, ties to even); a block whose
 *   maximum is below 2^-100 contributes nothing;
 *   out = sum_j P^_j v^_j / sum_j p_j  (bf16; zero rows for users with no keys).
 * Both products run on the block-scaled FP8 matrix instruction with fp32
 * accumulation; long key ranges are split and merged as in the bf16 path.
 *
 * ikbo_mx_create: a handle owning the work lists (pinned host memory, 16
 *   buffers used in turn, as for plans; a call on another stream than the
 *   handle's previous one first waits for that stream) and the split partials
 *   (64 KB + 2 KB per slot).
 * ikbo_attn_fwd_mxfp8: user_offsets [n_users + 1] and cand_to_user [n_cand]
 *   are HOST int32 arrays; the tensors are device arrays, row-major uint8:
 *     q_codes [n_cand, n_q, H, d]   q_scales [n_cand, n_q, H, d/32]
 *     k_codes [T, H, d]             k_scales [T, H, d/32]
 *     v_codes [T, H, d]             v_scales [NVB, H, d]
 *   with T = user_offsets[n_users], NVB = sum_u ceil(L_u / 32) (user u's
 *   blocks follow user u-1's; block b of u covers its keys 32b .. 32b+31, for
 *   every head and column); out [n_cand, n_q, H, d] bf16.  Codes and out must
 *   be 16-byte aligned, scales 4-byte aligned; d must be 128.  NaN codes or
 *   scales are the caller's to avoid (they propagate).  Enqueues one kernel (two
 *   when key ranges are split) on `stream` and returns without synchronising
 *   (it may wait for the call before last on the same handle to finish reading
 *   its work list).  Errors (INVALID_ARG: null or misaligned tensors, out
 *   aliasing an input, bad sizes, non-finite scale; BAD_OFFSETS; BAD_MAPPING;
 *   UNSUPPORTED: d != 128) launch nothing.  Calls on one handle must be
 *   ordered on one stream.
 * ikbo_mx_info: info[0] work items, info[1] split groups, info[2] workgroups of
 *   the last call.
 * ikbo_mx_timing / _timing_read: per-call durations of the attention kernel
 *   and of the merge (0 when nothing was split), from events stamped by the
 *   dispatches (at most 4096 calls between resets).
 * ikbo_mx_destroy: frees the handle after synchronising its device.
 */
int ikbo_mx_create(void** mx);
int ikbo_attn_fwd_mxfp8(void* mx, const int32_t* user_offsets, const int32_t* cand_to_user, int32_t n_users,
                        int32_t n_cand, int32_t n_q, int32_t H, int32_t d, float scale, const void* q_codes,
                        const void* q_scales, const void* k_codes, const void* k_scales, const void* v_codes,
                        const void* v_scales, void* out, void* stream);
int ikbo_mx_info(void* mx, int64_t* info, int32_t n_info);
int ikbo_mx_timing(void* mx, int32_t enable);
int ikbo_mx_timing_read(void* mx, float* attn_ms, float* merge_ms, int32_t max_n, int32_t* n);
void ikbo_mx_destroy(void* mx);

/*
 * Introspection of a built plan (host values), for tests and measurement:
 * info[0] work items, [1] grid of the persistent launch, [2] split groups,
 * [3] partial-result slots, [4] bytes of the split-KV workspace, [5] target
 * row tiles, [6] self row tiles, [7] compute units, [8] kernel (0 fp32, 1 bf16
 * eight-wave, 2 bf16 4-wave, 4 bf16 4-wave visiting each item's key tiles last
 * to first).  Writes the first min(n_info, 9) values.
 */
int ikbo_plan_info(void* plan, int64_t* info, int32_t n_info);

#ifdef __cplusplus
}
#endif

#endif /* IKBO_H_ */
