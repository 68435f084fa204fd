/*
 * star_attn.h -- C ABI of the MI355X (gfx950) Star Attention hot path.
 *
 * Star Attention runs long-context inference in two phases:
 *   Phase 1 (context encoding): the context is cut into blocks of b tokens;
 *     every block after the first is prefixed with an anchor block (the
 *     first block, at its original position ids) and attends causally within
 *     that augmented block only; the anchor's KV is then discarded.
 *   Phase 2 (query and generation): query and generated tokens attend to
 *     every cached token; each KV partition ("host") produces a local output
 *     and a log-sum-exp, and an exact online-softmax merge combines them.
 * Sources: Pith review of "Star Attention: Efficient LLM Inference over Long
 * Sequences" ("What carries the argument", "Referee Report", "Circularity
 * Check", "Assumptions & free parameters"); the atlas.scime.ai summary of
 * the same paper ("Approach"); the NVIDIA/Star-Attention repository README
 * (graphcanon record).  On one GPU the hosts are KV partitions resident in
 * one HBM.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are described by star_tensor: a [B, H, S, D] view with element
 *   strides sB, sH, sS and unit stride along D.  Data must be device memory
 *   aligned to 16 bytes, and every stride times the element size must be a
 *   multiple of 16 bytes.
 * - Q/K/V are bf16 (STAR_BF16); fp32 (STAR_F32) inputs are accepted by
 *   Phase 1 and Phase 2 and rounded to bf16 (nearest-even) when loaded.
 * - GQA: query head h reads KV head h / g, g = Hq / Hkv (g <= 16).
 * - Head dim D is 64 or 128.
 * - Position ids: a context token's position is its index in the context;
 *   the KV cache is position-contiguous, so cache index == position.
 * - lse values are natural-log log-sum-exp of the scaled scores (scale is
 *   passed by the caller, normally 1/sqrt(D)).  A row that sees no key has
 *   o = 0 and lse = -inf.
 * - Ownership: the caller allocates and owns every buffer.  No entry point
 *   allocates, frees or synchronises, with one exception in the attention
 *   layer's calls: star_context_create allocates the context and its fixed
 *   rocBLAS workspace (star_context_destroy frees them); star_linear then
 *   allocates nothing.  Work is enqueued on `stream` (a
 *   hipStream_t passed as void*; NULL = the null stream) and the call returns
 *   without waiting.  The library holds no mutable global state apart from
 *   star_decode_step_noalloc's per-GPU scratch array (see there), so the
 *   other calls are reentrant and thread-safe.
 * - Errors: arguments are validated on the host before anything is
 *   enqueued; a negative star_status is returned and nothing runs.  A launch
 *   failure reported by the HIP runtime returns STAR_ERR_HIP.  No C++
 *   exception crosses this boundary.  Inputs holding NaN or Inf give
 *   unspecified (but memory-safe) results.
 */
#ifndef STAR_ATTN_H
#define STAR_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STAR_OK = 0,
  STAR_ERR_NULL = -1,        /* a required pointer is NULL */
  STAR_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
  STAR_ERR_DTYPE = -3,       /* unsupported dtype or dtype combination */
  STAR_ERR_ALIGN = -4,       /* data or stride not 16-byte aligned */
  STAR_ERR_UNSUPPORTED = -5, /* valid request this build does not serve */
  STAR_ERR_HIP = -6,         /* the HIP runtime reported a launch error */
  STAR_ERR_BLAS = -7         /* the BLAS library (rocBLAS) reported an error */
} star_status;

typedef enum { STAR_BF16 = 0, STAR_F32 = 1 } star_dtype;

/* [B, H, S, D] device tensor; strides in elements; D has unit stride. */
typedef struct {
  void* data;
  int32_t dtype; /* star_dtype */
  int32_t reserved;
  int64_t B, H, S, D;
  int64_t sB, sH, sS;
} star_tensor;

/* Largest number of KV partitions star_phase2_partial accepts, and of
   blocks star_phase1_prefix accepts. */
#define STAR_MAX_PARTS 128
/* Split chunks of a partition are whole multiples of this many keys. */
#define STAR_SPLIT_ALIGN 64
/*
 * Phase-1 scheduling workspace: int32 count of the optional `sched` buffer
 * of the Phase-1 calls (device memory, 4-byte aligned, owned by the
 * caller).  With it, the bf16 D = 128 kernel hands out its work items from
 * per-XCD queues kept in that buffer: an XCD that runs faster than the
 * others (their clocks differ by several percent under a full load) takes
 * over their remaining items instead of idling at the end.  NULL keeps a
 * fixed share per XCD.  Results are identical either way (items are
 * independent).  The call clears the buffer itself, on `stream`, before
 * its kernel uses it; the contents are scratch afterwards.  Two calls that
 * may run at the same time (different streams) must not share a buffer.
 * The other Phase-1 kernels (D = 64, fp32 inputs) ignore it.
 */
#define STAR_SCHED_INTS 16

/*
 * Rotary position embedding at original position ids (rotate-half form).
 * Pair (j, j + D/2) of a row at position p is rotated by the angle
 * p * theta_j, theta_j = base^(-2j/D): the anchor block keeps the first
 * block's positions and every token keeps its own (Pith review of Star
 * Attention, "What carries the argument"; atlas.scime.ai summary, anchor
 * position-id ablation).  Everything before the one rounding to the
 * output dtype is fp64: the angle is the IEEE product p * theta_j (theta_j
 * as star_rope_freqs returns it), cos/sin are fp64, the pair is rotated in
 * fp64 and rounded once to nearest even.  The stored value is therefore the
 * exact rotation of the input rounded once, up to fp64 rounding (it can
 * differ only where that value lies within a few fp64 ulps of a rounding
 * midpoint).  Every kernel that rotates (star_kv_append,
 * star_decode_prepare, star_phase1_rope, star_decode_step) uses the same
 * arithmetic, so they store the same bits for the same position.
 *
 *   x_in   [B, H, S, D] bf16 or fp32.
 *   x_out  same shape and dtype; may alias x_in exactly (in place).
 *   pos    device int64 [S] position of each row, or NULL for pos0 + s.
 * Returns STAR_OK or a negative star_status.
 */
int star_rope_apply(const star_tensor* x_in, const star_tensor* x_out,
                    const int64_t* pos, int64_t pos0, double base,
                    void* stream);

/*
 * The RoPE frequencies every rotating entry point uses (host only, no GPU
 * call): inv_freq[j] = theta_j = base^(-2j/D) for j < D/2, evaluated in
 * extended precision and rounded once to fp64 (the fp64 value nearest the
 * exact power).
 *   D         head dim: 16 <= D <= 128, D % 16 == 0 (else
 *             STAR_ERR_UNSUPPORTED).
 *   base      > 1 and finite (else STAR_ERR_SHAPE).
 *   inv_freq  host double [D / 2] output (else STAR_ERR_NULL).
 */
int star_rope_freqs(int64_t D, double base, double* inv_freq);

/*
 * Append new tokens' KV to a position-contiguous cache: the query host
 * stores the query and generated tokens' KV (Pith review of Star Attention,
 * "What carries the argument").  Row t of k_new is rotated at position
 * pos0 + t (when rope != 0) and written to k_cache row slot0 + t; row t of
 * v_new is copied to v_cache row slot0 + t.
 *
 *   k_new, v_new      [B, Hkv, T, D] bf16.
 *   k_cache, v_cache  [B, Hkv, S, D] bf16, slot0 + T <= S.
 */
int star_kv_append(const star_tensor* k_new, const star_tensor* v_new,
                   const star_tensor* k_cache, const star_tensor* v_cache,
                   int64_t slot0, int64_t pos0, double base, int32_t rope,
                   void* stream);

/*
 * One generated token's (or a few query tokens') preparation in one launch:
 * the new query rows are rotated at positions pos0 + t into q_out, and the
 * new K/V rows are appended to the cache exactly as star_kv_append does
 * (k rotated at pos0 + t into k_cache row slot0 + t, v copied).  Each
 * generated token repeats Phase 2 with its own query and cached KV (Pith
 * review of Star Attention, "What carries the argument" and "Core claim").
 *
 *   q_new, q_out      [B, Hq, T, D] bf16 (q_out may alias q_new exactly).
 *   k_new, v_new      [B, Hkv, T, D] bf16.
 *   k_cache, v_cache  [B, Hkv, S, D] bf16, slot0 + T <= S.
 * With rope == 0 the rows are copied unrotated.
 */
int star_decode_prepare(const star_tensor* q_new, const star_tensor* q_out,
                        const star_tensor* k_new, const star_tensor* v_new,
                        const star_tensor* k_cache, const star_tensor* v_cache,
                        int64_t slot0, int64_t pos0, double base, int32_t rope,
                        void* stream);

/*
 * Phase 1: anchor-block blockwise-local causal attention.
 * The context (length L = q->S) is cut into blocks [i*b, min((i+1)*b, L)).
 * Rows of the first block attend causally within it.  A row at position p
 * of block i >= 1 attends to the anchor keys [0, anchor_len) (the first
 * tokens at their original positions; their K/V are the first block's K/V,
 * read in place) and to its own block's keys up to and including p.
 * Anchor rows are never recomputed or output for later blocks (Pith review
 * of Star Attention, "What carries the argument" and Referee Report minor
 * comment on Section 2.1; atlas.scime.ai summary, "Approach").
 * anchor_len = block_b is the method; 0 <= anchor_len < block_b gives the
 * pages' smaller-anchor and no-anchor ablations.
 *
 *   q      [B, Hq, L, D] bf16 or fp32, rotated.
 *   k, v   [B, Hkv, L, D], same dtype as q, k rotated.
 *   o      [B, Hq, L, D] bf16 output.
 *   lse    fp32 [B, Hq, L] contiguous output, or NULL.
 *   sched  device int32 [STAR_SCHED_INTS] scheduling workspace, or NULL
 *          (see STAR_SCHED_INTS); STAR_ERR_ALIGN unless 4-byte aligned.
 */
int star_phase1_blocklocal(const star_tensor* q, const star_tensor* k,
                           const star_tensor* v, int64_t block_b,
                           int64_t anchor_len, float scale,
                           const star_tensor* o, float* lse, int32_t* sched,
                           void* stream);

/*
 * Phase 1 with the RoPE of Q fused in: as star_phase1_blocklocal, but q
 * holds the un-rotated query rows and the kernel rotates row r at its
 * original position r (rotate-half, theta_j = base^(-2j/D); Pith review of
 * Star Attention, "What carries the argument": original position ids), as
 * star_rope_apply would, before attending.  k must already be rotated (it
 * is the KV cache).  The rotation is star_rope_apply's (same fp64 angle
 * reduction, sin/cos and rounding), so the output equals that of
 * star_rope_apply followed by star_phase1_blocklocal bit for bit.  Saves
 * the separate pass over Q and its rotated copy.
 *   base   > 1.
 * Returns STAR_ERR_UNSUPPORTED unless q/k/v are bf16 with D = 128 (the
 * kernel that carries the rotation).  sched as for star_phase1_blocklocal.
 */
int star_phase1_rope(const star_tensor* q, const star_tensor* k,
                     const star_tensor* v, int64_t block_b,
                     int64_t anchor_len, double base, float scale,
                     const star_tensor* o, float* lse, int32_t* sched,
                     void* stream);

/*
 * Phase 1 with an explicit per-block prefix in place of the anchor.
 * Rows of block i (i = 0 .. nblocks-1, blocks as in
 * star_phase1_blocklocal) attend to every row of
 * [pk, pv][prefix_start[i], prefix_start[i] + prefix_len[i]) -- all of it,
 * the prefix precedes the block -- and then to their own block's keys up to
 * and including themselves.  The prefix rows are read, never output.
 * This one form covers the variants the pages describe:
 *  - the anchor itself: pk = k, pv = v, start 0, length a for i >= 1, 0 for
 *    block 0 (what star_phase1_blocklocal computes);
 *  - the anchor at other position ids (atlas.scime.ai summary, "Measured
 *    effects reported in the paper"): the anchor keys re-rotated per block
 *    (star_rope_apply with a position list) into pk;
 *  - other anchor content (same ablation table): any rows in pk/pv;
 *  - Pulsar's 64-token sink plus the Max-IDF summaries of all earlier
 *    blocks, at their original position ids (Pith review of Pulsar
 *    Attention, "What carries the argument"): rows gathered with
 *    star_gather_rows, table from star_pulsar_prefix.
 *
 *   q, k, v        as for star_phase1_blocklocal (L = q->S = k->S).
 *   pk, pv         [B, Hkv, R, D], same dtype as q (may be k and v).
 *   prefix_start   host int64 [nblocks], prefix_len host int64 [nblocks]:
 *                  0 <= start, 0 <= len, start + len <= R.
 *   nblocks        must equal ceil(L / block_b), at most STAR_MAX_PARTS.
 *   o, lse, sched  as for star_phase1_blocklocal.
 */
int star_phase1_prefix(const star_tensor* q, const star_tensor* k,
                       const star_tensor* v, const star_tensor* pk,
                       const star_tensor* pv, const int64_t* prefix_start,
                       const int64_t* prefix_len, int32_t nblocks,
                       int64_t block_b, float scale, const star_tensor* o,
                       float* lse, int32_t* sched, void* stream);

/*
 * Row gather: dst[b, h, r, :] = src[b, h, rows[r], :] for r < dst->S.  A
 * row index outside [0, src->S) yields a zero row (no fault).  Used to
 * assemble a prefix from context rows at their original positions (Pith
 * review of Pulsar Attention, "What carries the argument": the sink and
 * summary tokens keep their global position ids, so their rotated K/V are
 * the context's own rows).
 *
 *   src   [B, H, S, D] bf16 or fp32.
 *   rows  device int64 [dst->S] (may be NULL when dst->S == 0).
 *   dst   [B, H, R, D], same B, H, D and dtype as src; must not overlap src.
 */
int star_gather_rows(const star_tensor* src, const int64_t* rows,
                     const star_tensor* dst, void* stream);

/*
 * Pulsar's Phase-1 prefix (host-side integer work, no GPU call): Max-IDF
 * chunk summaries and the per-block prefix table (Pith review of Pulsar
 * Attention, "What carries the argument", "Core claim", "Assumptions & free
 * parameters").  With n = ceil(L / block_b) blocks, df(t) = number of
 * blocks containing token t and IDF(t) = log(n / max(df(t), 1)) (fp64):
 *  - every block is cut into chunks of chunk_m tokens (the last may be
 *    shorter); score(C) = max over t in C of IDF(t);
 *  - summary i = the k best-scoring chunks of block i (equal scores: the
 *    earlier chunk first), listed in positional order; in block 0 the chunks
 *    that overlap the sink are not candidates;
 *  - rows = [0, s) ++ summary 0 ++ ... ++ summary n-2, with s =
 *    min(sink, block_b, L) the attention sink;
 *  - block 0 has no prefix (prefix_len[0] = 0); block i >= 1 has
 *    prefix_start[i] = 0 and prefix_len[i] = s + |summary 0| + ... +
 *    |summary i-1|: the sink and the summaries of all earlier blocks.
 *
 *   tokens        host int32 [L] token ids.
 *   rows          host int64 [rows_cap] output; *n_rows receives the count.
 *                 If rows_cap is too small, *n_rows is set to the count
 *                 needed and STAR_ERR_SHAPE is returned.
 *   prefix_start, prefix_len  host int64 [nblocks] outputs;
 *                 nblocks must equal n.
 * chunk_m >= 1, sink >= 0, k >= 0.
 */
int star_pulsar_prefix(const int32_t* tokens, int64_t L, int64_t block_b,
                       int32_t chunk_m, int32_t sink, int32_t k,
                       int64_t* rows, int64_t rows_cap, int64_t* n_rows,
                       int64_t* prefix_start, int64_t* prefix_len,
                       int32_t nblocks);

/*
 * Phase 2 partials: local attention of query rows over each KV partition.
 * Partition j covers cache rows [part_offsets[j], part_offsets[j+1]); the
 * last partition is the query host and also holds the query/decode tokens'
 * KV.  Each partition is cut into `splits` chunks of
 * c_j = roundup(ceil(n_j / splits), STAR_SPLIT_ALIGN) keys; chunk s covers
 * [off_j + s*c_j, min(off_j + (s+1)*c_j, off_{j+1})) and may be empty.
 * Query row r sits at position q_pos0 + r and sees cache row c iff
 * c <= q_pos0 + r.  For every chunk the call writes the chunk-local
 * attention output (normalised within the chunk) and its lse: one vector
 * and one scalar per token (Pith review of Star Attention, "Core claim",
 * "Circularity Check").
 *
 *   q             [B, Hq, Lq, D] bf16 or fp32, rotated.
 *   k_cache/v_cache [B, Hkv, S, D], same dtype as q.
 *   part_offsets  host int64 [P + 1], non-decreasing, last <= S.
 *   o_part        device fp32 [P*splits, B, Hq, Lq, D] contiguous, chunk
 *                 index j*splits + s.
 *   lse_part      device fp32 [P*splits, B, Hq, Lq] contiguous.
 * 1 <= P <= STAR_MAX_PARTS, 1 <= splits <= 1024.
 */
int star_phase2_partial(const star_tensor* q, const star_tensor* k_cache,
                        const star_tensor* v_cache,
                        const int64_t* part_offsets, int32_t P, int32_t splits,
                        int64_t q_pos0, float scale, float* o_part,
                        float* lse_part, void* stream);

/*
 * Exact online-softmax (log-sum-exp) merge of N partials per row:
 * s = log(sum_n exp(s_n)), A = sum_n exp(s_n - s) * A_n; partials with
 * s_n = -inf carry no weight (Pith review of Star Attention, Referee Report
 * minor comment on Algorithm 2; "Circularity Check").
 *
 *   o_part    fp32 [N, B, Hq, Lq, D] contiguous (star_phase2_partial's
 *             layout; R = B * Hq * Lq rows per partial).
 *   lse_part  fp32 [N, B, Hq, Lq] contiguous.
 *   o         [B, Hq, Lq, D] bf16 or fp32 output, any strides; its sizes
 *             must equal the B, Hq, Lq, D given (else STAR_ERR_SHAPE).
 *   lse       fp32 [B, Hq, Lq] contiguous output, or NULL.
 * 1 <= N <= 65536; D is 64 or 128.
 */
int star_lse_merge(const float* o_part, const float* lse_part, int32_t N,
                   int64_t B, int64_t Hq, int64_t Lq, int64_t D,
                   const star_tensor* o, float* lse, void* stream);

/*
 * One whole decode step of one generated token: the token's query and key
 * are rotated at `pos` (when rope != 0), its K/V row is appended at cache
 * row `slot`, and the split-KV partials over every partition are computed
 * exactly as star_phase2_partial does (Lq = 1, q_pos0 = pos) -- all in one
 * launch -- followed by the star_lse_merge of those partials.  Each
 * generated token attends globally to every cached token (Pith review of
 * Star Attention, "What carries the argument", "Core claim" and
 * "Circularity Check").  The rotation is star_rope_apply's (fp64, one
 * rounding), so the appended K row equals star_kv_append's bit for bit.
 * The cache is position-contiguous: the token's row is its position, so
 * slot must equal pos (else STAR_ERR_SHAPE); it sees every cache row
 * c <= pos of the partitions, including its own.
 *
 *   q_new             [B, Hq, 1, D] bf16, un-rotated.
 *   k_new, v_new      [B, Hkv, 1, D] bf16 (k un-rotated).
 *   k_cache, v_cache  [B, Hkv, S, D] bf16; row `slot` is overwritten.
 *   part_offsets      host int64 [P + 1] as for star_phase2_partial;
 *                     part_offsets[0] <= slot < part_offsets[P].
 *                     Rows past slot are never read, so they may hold
 *                     anything (unwritten cache rows).
 *   o_part, lse_part  device fp32 workspaces of star_phase2_partial's sizes
 *                     ([P*splits, B, Hq, 1, D] and [P*splits, B, Hq]);
 *                     they hold the chunk partials afterwards.
 *   o                 [B, Hq, 1, D] bf16 or fp32 merged output.
 *   lse               fp32 [B, Hq] contiguous merged lse, or NULL.
 */
int star_decode_step(const star_tensor* q_new, const star_tensor* k_new,
                     const star_tensor* v_new, const star_tensor* k_cache,
                     const star_tensor* v_cache, int64_t slot, int64_t pos,
                     double base, int32_t rope, const int64_t* part_offsets,
                     int32_t P, int32_t splits, float scale, float* o_part,
                     float* lse_part, const star_tensor* o, float* lse,
                     void* stream);

/*
 * star_decode_step with the token's position in device memory, so that one
 * recorded sequence of launches (a captured HIP graph) serves every
 * generated token: the host arguments stay the same from step to step.
 * Each generated token attends globally to every cached token (Pith review
 * of Star Attention, "Core claim"); the step is star_decode_step's at
 * slot = pos = *pos, read at the start of the step, and the step's second
 * launch (the merge) then adds one to *pos.
 *   pos               device int64, 8-byte aligned, one position for every
 *                     sequence of the batch (they decode in lockstep, as
 *                     with star_decode_step).  When the step runs,
 *                     part_offsets[P - 1] <= *pos < part_offsets[P] must
 *                     hold; the last partition then ends right after the
 *                     token (rows *pos + 1 .. are never read).  For any
 *                     other value the step writes no cache row, its
 *                     outputs are o = 0 and lse = -inf, and *pos is still
 *                     advanced.
 *   part_offsets      host int64 [P + 1]: partition starts, and in
 *                     part_offsets[P] the end bound of the positions this
 *                     call may be replayed at (<= S).  The split chunks of
 *                     the last partition follow its current length.
 *   Other arguments, workspaces and errors are star_decode_step's, except
 *   STAR_ERR_NULL for pos == NULL, STAR_ERR_ALIGN for a misaligned pos,
 *   and STAR_ERR_SHAPE when part_offsets[P - 1] >= part_offsets[P].
 *   No allocation; two launches on `stream` and nothing on the host that
 *   depends on the position, so the call can be captured.  Steps that share
 *   *pos must run in order on one stream.
 */
int star_decode_step_devpos(const star_tensor* q_new, const star_tensor* k_new,
                            const star_tensor* v_new, const star_tensor* k_cache,
                            const star_tensor* v_cache, int64_t* pos, double base,
                            int32_t rope, const int64_t* part_offsets, int32_t P,
                            int32_t splits, float scale, float* o_part, float* lse_part,
                            const star_tensor* o, float* lse, void* stream);

/*
 * star_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call without the o_part / lse_part workspaces.  The
 * split-KV partials live in a file-scope device array of
 * STAR_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends; its address on the current device is looked up once per
 * device.  The call allocates nothing and frees nothing.
 *   Arguments, semantics and errors are star_decode_step's; in addition
 *   STAR_ERR_UNSUPPORTED when the partials, P * splits * B * Hq rows of
 *   D + 1 floats, do not fit the array (about 8000 rows at D = 128), and
 *   STAR_ERR_HIP when the array's address cannot be obtained.
 *   Every call on one GPU uses that GPU's one array, and each call
 *   overwrites every partial it reads before reading it: calls that may
 *   overlap on one GPU (different streams, different threads) race and must
 *   not be issued.
 */
#define STAR_NOALLOC_SCRATCH_BYTES (4 << 20)
int star_decode_step_noalloc(const star_tensor* q_new, const star_tensor* k_new,
                             const star_tensor* v_new, const star_tensor* k_cache,
                             const star_tensor* v_cache, int64_t slot, int64_t pos,
                             double base, int32_t rope, const int64_t* part_offsets,
                             int32_t P, int32_t splits, float scale,
                             const star_tensor* o, float* lse, void* stream);

/*
 * The attention layer around Phase 1 (the Llama-3 attention block of the
 * pages' HuggingFace models: graphcanon record of NVIDIA/Star-Attention,
 * README): out = x + Attn(rope(RMSNorm(x) W^T)) Wo^T.  Phase 1 of a
 * multi-layer model is this layer applied to all L tokens at every layer:
 * the anchor is causal and first in every augmented block, so its hidden
 * states, and its K/V, equal block 1's at every layer (Pith review of Star
 * Attention, "What carries the argument").
 *
 * The projections are plain GEMMs and run in rocBLAS; a star_context owns
 * the rocBLAS handle and a device workspace of STAR_BLAS_WORKSPACE_BYTES
 * handed to rocBLAS, so that star_linear never allocates.  Create one per
 * thread that issues star_linear calls, on the device they will run on
 * (star_context_create allocates; it is not a hot call: STAR_ERR_HIP if the
 * workspace cannot be allocated, STAR_ERR_BLAS if rocBLAS fails), and
 * destroy it when done.  Calls with one context must not run concurrently
 * from two threads or streams (they share the workspace).
 */
#define STAR_BLAS_WORKSPACE_BYTES (64 << 20)
typedef struct star_context star_context;

int star_context_create(star_context** ctx);
int star_context_destroy(star_context* ctx);   /* NULL is a no-op */

/*
 * RMSNorm of every row: y = x / sqrt(mean(x^2) + eps) * gamma, the sum of
 * squares in fp32, one rounding to bf16.
 *   x, y   [B, H, S, D] bf16 (rows of length D, D % 8 == 0); y may alias x
 *          exactly.
 *   gamma  device bf16 [D], 16-byte aligned.
 */
int star_rmsnorm(const star_tensor* x, const void* gamma, float eps,
                 const star_tensor* y, void* stream);

/*
 * y = x w^T (+ residual): bf16 operands, fp32 accumulation, bf16 result.
 *   x         [1, 1, M, K] (row stride x->sS >= K).
 *   w         [1, 1, N, K] (the [out, in] weight layout).
 *   residual  [1, 1, M, N] or NULL; may be y itself.
 *   y         [1, 1, M, N].
 * Every row stride times 2 bytes is a multiple of 16.  Returns
 * STAR_ERR_BLAS if rocBLAS fails.
 */
int star_linear(star_context* ctx, const star_tensor* x, const star_tensor* w,
                const star_tensor* residual, const star_tensor* y, void* stream);

/*
 * Measurement aid, not a step of the method: a plain streaming read of
 * `bytes` bytes of device memory at `src` (each byte once, 16-byte
 * nontemporal loads).
 * Workgroup i reads bytes [i, i + 1) * bytes / workgroups and writes the XOR
 * of the 32-bit words it read to out[i], so the XOR of out[0 .. workgroups)
 * is the XOR of every word of the buffer.  Its rate is the practical
 * ceiling for the HBM-bound decode kernel on the GPU it runs on.
 *   src         device, 16-byte aligned.
 *   bytes       > 0, a multiple of workgroups * 32768.
 *   workgroups  1 .. 65536.
 *   out         device uint32 [workgroups], 4-byte aligned.
 * Errors: STAR_ERR_NULL, STAR_ERR_ALIGN, STAR_ERR_SHAPE (sizes above).
 */
int star_stream_read(const void* src, int64_t bytes, int32_t workgroups,
                     uint32_t* out, void* stream);

/* Human-readable name of a star_status value (static storage). */
const char* star_status_string(int status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int star_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STAR_ATTN_H */
