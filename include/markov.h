/*
 * markov.h -- C ABI of the MI355X (gfx950) DSpark sequential Markov
 * draft-sampling step.
 *
 * What one call computes (the pages' definition):
 *   For each draft step s = 0..k-1 and request row r, with t the token that
 *   feeds the step (prev[r] at s = 0, else the token step s-1 sampled):
 *     emb   = w1[min_u64(t, V-1)]                          gather, clamped
 *     b[v]  = bf16( sum_j emb[j] * w2[v][j] )              fp32 dot, one rounding
 *     x[v]  = bf16( base[r][s][v] + b[v] )                 fp32 add, to bf16
 *     c[v]  = bf16( cap > 0 ? cap*tanh(mult*x*RN32(1/cap)) : mult*x )
 *     cache[r][s][v] = c[v]
 *     key[v] = T != 0 ? RN32(RN32(c/T) - log(-log1m(u)))  :  c
 *              u from MurmurHash3(seed, step, position, v)
 *     tokens[r][s] = the first NaN key, else the lowest id of the largest key
 *   Sources (vLLM API pages): "vllm.models.kimi_k3.nvidia.specialized_decode.
 *   drafter.markov" (module docstring: the exactness paragraph; `_gumbel_key`,
 *   `_loop_rest`), "vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.
 *   draft.markov" (module docstring; `_logit`, `_gumbel`, `_murmur_prefix`,
 *   `_combine`, `_w1_row`, `markov_step`), "vllm.models.deepseek_v41.amd.ops.
 *   fused_markov" (module docstring).
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers are HIP device memory owned by the
 *     caller; the library never frees or keeps them. `stream` is a hipStream_t
 *     (NULL = the default stream).
 *   - Nothing is allocated and no host synchronisation happens inside
 *     markov_sample_sequential; it only enqueues kernels on `stream`, so it
 *     can be captured into a HIP graph.
 *   - Errors are detected on the host only and returned as a negative
 *     MARKOV_ERR_* code (0 = success); nothing is enqueued on an error.
 *     Device data is never validated: an out-of-range token reads the last
 *     w1 row (the pages' `_w1_row` clamp), NaN logits flow through the total
 *     order, and a NaN temperature makes every key NaN.
 */
#ifndef MARKOV_H_
#define MARKOV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* markov_stream_t; /* a hipStream_t */

/* Shape of one loop. rows: request rows; vocab: V (a multiple of 8);
 * rank: R, a power of two in [16, 512] (the gate of the kimi_k3 page's
 * `why_not`); mult: the output multiplier; softcap: the soft cap, <= 0 for
 * none (the muse_spark page's `_logit` output transform). */
typedef struct markov_shape {
  int32_t rows;
  int32_t vocab;
  int32_t rank;
  float mult;
  float softcap;
} markov_shape_t;

enum {
  MARKOV_OK = 0,
  MARKOV_ERR_NULL = -1,        /* a required pointer is NULL */
  MARKOV_ERR_SHAPE = -2,       /* rows < 1, vocab < 1 or not a multiple of 8, k < 1 */
  MARKOV_ERR_RANK = -3,        /* rank not a power of two in [16, 512] */
  MARKOV_ERR_ALIGN = -4,       /* a bf16 array not 16-byte aligned */
  MARKOV_ERR_ROWS = -5,        /* rows above what the rank's LDS budget holds */
  MARKOV_ERR_WORKSPACE = -6,   /* workspace smaller than markov_workspace_bytes */
  MARKOV_ERR_HIP = -7,         /* a HIP runtime call failed */
  MARKOV_ERR_VOCAB = -8        /* vocab (or a shard's vocab_total) above MARKOV_MAX_VOCAB */
};

/* The largest vocabulary the library takes: token ids and in-slab offsets
   are 32-bit integers, with room for one vocabulary slab past the end. */
#define MARKOV_MAX_VOCAB 0x7fff0000

/* The most rows one call takes at a given rank (at most 512; the embedding
 * rows are staged in LDS next to per-row data, within 160 KiB). */
int32_t markov_max_rows(int32_t rank);

/* Bytes of device workspace one loop of this shape needs (independent of
 * k), in this order:
 *   - the noise bound tables, 25856 bytes: 2176 per-bucket lines as (A, B)
 *     binary32 pairs, then 2112 binary32 constants;
 *   - the output-transform table, 65792 bytes: a 256-byte stamp (a magic
 *     word, then the bits of the mult and softcap it was built for), then
 *     32768 bf16 entries, entry i holding the cached value of the bf16 sum
 *     whose bits are i (the transform is odd, so negative sums take the
 *     entry of their magnitude with the sign flipped);
 *   - a 256-byte block holding the last step's completion count (zero
 *     between calls);
 *   - the winner slots: for each of three steps in turn, 8 per-row arrays of
 *     packed (key, id) maxima (workgroups publish into 8 groups; a step's
 *     winner is the largest over them), 192 bytes per row. */
size_t markov_workspace_bytes(const markov_shape_t* shape, int32_t k);

/* Prepare a workspace once after allocating it (enqueued on `stream`): the
 * noise bound tables are copied in, the transform table is built on the host
 * for shape->mult and shape->softcap (only with a soft cap; shape may be
 * NULL, then no transform table is stamped) and copied in, and the ticket
 * and the slot arrays are zeroed. Every call of markov_sample_sequential leaves it so
 * again, so it is reused as is; it must not be shared by two calls in flight
 * at once. 16-byte aligned. A call whose (mult, softcap) differ from the
 * stamp still gives the same results within the stated tolerance: it
 * evaluates the transform itself instead of looking it up. */
int markov_workspace_init(void* workspace, size_t bytes, const markov_shape_t* shape,
                          markov_stream_t stream);

/* NULL when this shape and k are supported, else why not (a static string);
 * mirrors the pages' fallback gates (kimi_k3 `why_not`, deepseek_v41
 * `_why_not`) for what a call can check. */
const char* markov_why_not(const markov_shape_t* shape, int32_t k);

/*
 * The k-step loop: one kernel launch per draft step on `stream`.
 *   base_logits  device, bf16 [rows, k, V] contiguous        (read)
 *   w1, w2       device, bf16 [V, R] contiguous row-major    (read)
 *   prev         device, int64 [rows]: the token feeding step 0 (read)
 *   seeds        device, int64 [rows]: per-request seed      (read)
 *   positions    device, int64 [rows, k]: sample position of each step;
 *                the noise hashes positions[r][s] - 1 + 2^30 (read)
 *   k            number of draft steps, >= 1
 *   temperature  device, fp32 [rows]; 0 (or -0) means plain argmax (read)
 *   cache        device, bf16 [rows, k, V] contiguous        (write)
 *   tokens       device, int64 [rows, k] contiguous          (write)
 *   stream       hipStream_t
 *   shape        host pointer (rows, V, R, mult, softcap)
 *   workspace    device, zeroed once by markov_workspace_init
 *   workspace_bytes  its size, >= markov_workspace_bytes(shape, k)
 * base_logits, w1, w2 and cache must be 16-byte aligned; cache must not
 * overlap base_logits.
 */
int markov_sample_sequential(const void* base_logits, const void* w1, const void* w2,
                             const int64_t* prev, const int64_t* seeds,
                             const int64_t* positions, int32_t k, const float* temperature,
                             void* cache, int64_t* tokens, markov_stream_t stream,
                             const markov_shape_t* shape, void* workspace,
                             size_t workspace_bytes);

/*
 * Step `step` (0 <= step < k) of the same loop alone: one kernel launch that
 * feeds on prev (step 0) or on the previous step's winners (kept in the
 * workspace), writes cache[:, step, :] and tokens[:, step-1]; the launch of
 * the last step (step = k-1) also writes tokens[:, k-1] and re-zeroes the
 * workspace's slots. Arguments and errors as markov_sample_sequential;
 * calling it for step = 0..k-1 in order is that loop.
 */
int markov_sample_step(const void* base_logits, const void* w1, const void* w2,
                       const int64_t* prev, const int64_t* seeds, const int64_t* positions,
                       int32_t k, int32_t step, const float* temperature, void* cache,
                       int64_t* tokens, markov_stream_t stream, const markov_shape_t* shape,
                       void* workspace, size_t workspace_bytes);

/*
 * markov_sample_sequential for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same loop and results, with the library's own workspace
 * instead of a caller's. Each GPU the library runs on holds one such
 * workspace, a file-scope device array of 190208 bytes, until the process
 * ends; it takes at most markov_noalloc_max_rows() rows (512), and a larger
 * shape fails with MARKOV_ERR_WORKSPACE. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine). The first call on a
 * device copies the noise bound tables into its workspace, and a call whose
 * (mult, softcap) differ from the last soft-capped call's copies that
 * transform table in (host-to-device copies on `stream`; the table is built
 * on the host once per (mult, softcap) and kept): make one such call outside
 * any graph capture first. Every call enqueues a small fill kernel that
 * clears the workspace's ticket and slots, then the k step launches. All
 * calls on one GPU share its workspace: calls that overlap in time on one
 * GPU (two streams, two host threads) race and must be serialised by the
 * caller. Other arguments and errors as markov_sample_sequential.
 */
int markov_sample_sequential_noalloc(const void* base_logits, const void* w1, const void* w2,
                                     const int64_t* prev, const int64_t* seeds,
                                     const int64_t* positions, int32_t k,
                                     const float* temperature, void* cache, int64_t* tokens,
                                     markov_stream_t stream, const markov_shape_t* shape);

/* The most rows markov_sample_sequential_noalloc takes. */
int32_t markov_noalloc_max_rows(void);

/*
 * The greedy loop: markov_sample_sequential with every row at temperature 0
 * (TensorRT Edge-LLM "DSpark kernels" page: `dsparkMarkovGreedyFusedStep`,
 * correction plus exact top-1 in one launch per step, the previous step's
 * winner read from packed orderable slots with no host round trip). Each
 * step's token is the first NaN, else the lowest id of the largest cached
 * logit. A specialised kernel: no temperatures, seeds or positions are read,
 * no noise is hashed, and NaN and -inf logits are ranked exactly in
 * registers, so nothing is read back.
 *   base_logits, w1, w2, prev, k, stream, shape, workspace, workspace_bytes
 *                as markov_sample_sequential
 *   cache        device bf16 [rows, k, V], or NULL: the corrected logits are
 *                not stored (the page's chain mode, which never
 *                materialises the row)
 *   tokens       device int64 [rows, k] (write)
 *   winners      device uint64 [rows, k], or NULL (write): each step's packed
 *                winner, the page's `greedySlots` format: the high word an
 *                unsigned image of the winning logit that orders as the
 *                total order (every NaN highest, -0 as +0), the low word the
 *                complement of the token id (so equal logits favour the
 *                lowest id); markov_greedy_finalize turns it into tokens
 * Errors as markov_sample_sequential (cache, if given, 16-byte aligned).
 */
int markov_greedy_sequential(const void* base_logits, const void* w1, const void* w2,
                             const int64_t* prev, int32_t k, void* cache, int64_t* tokens,
                             uint64_t* winners, markov_stream_t stream,
                             const markov_shape_t* shape, void* workspace,
                             size_t workspace_bytes);

/* Step `step` of the greedy loop alone (as markov_sample_step is to
 * markov_sample_sequential): writes cache[:, step, :] (if cache), and
 * tokens / winners of step-1, and of step k-1 when step = k-1. */
int markov_greedy_step(const void* base_logits, const void* w1, const void* w2,
                       const int64_t* prev, int32_t k, int32_t step, void* cache, int64_t* tokens,
                       uint64_t* winners, markov_stream_t stream, const markov_shape_t* shape,
                       void* workspace, size_t workspace_bytes);

/* tokens[i] = the token id of packed winner winners[i], i < n (Edge-LLM page:
 * `dsparkFinalizeGreedyDraftTokens`). Device arrays; one small kernel on
 * `stream`. n = 0 does nothing; NULL arrays or n < 0 are errors. */
int markov_greedy_finalize(const uint64_t* winners, int64_t n, int64_t* tokens,
                           markov_stream_t stream);

/* ---- E4M3 w2 (TensorRT Edge-LLM "DSpark kernels" page:
 * `dsparkQuantizeMarkovW2Fp8`, `dsparkMarkovGreedyFusedStepFp8`) ---------- */

/*
 * Quantize a bf16 w2 [V, R] to E4M3 codes with one FP16 scale per row: the
 * scale is RN16(rowAbsMax / 448), so each row spans the E4M3 range; code j is
 * the E4M3 nearest to the binary32 quotient w[j] / scale (ties to even,
 * saturating at +-448); a zero scale gives zero codes.
 *   w2         device bf16 [vocab, rank] (read)
 *   w2q        device uint8 [vocab, rank] (write), 16-byte aligned for the steps below
 *   w2_scales  device uint16 [vocab] FP16 bit patterns (write), 16-byte aligned likewise
 * One kernel on `stream` (a wave per row). Errors: NULL pointers, vocab < 1,
 * vocab above MARKOV_MAX_VOCAB, rank not a power of two in [16, 512].
 */
int markov_quantize_w2_fp8(const void* w2, uint8_t* w2q, uint16_t* w2_scales, int32_t vocab,
                           int32_t rank, markov_stream_t stream);

/*
 * markov_sample_sequential with the E4M3 w2 in place of the bf16 one: the
 * bias is bf16(RN32(scale[v] * sum_j emb[j] * value(w2q[v][j]))), the dot in
 * fp32 (the codes decode exactly to bf16 for the same MFMA contraction), the
 * scale applied once, then one rounding to bf16. Everything else as
 * markov_sample_sequential; w2q and w2_scales as markov_quantize_w2_fp8
 * writes them (16-byte aligned).
 */
int markov_sample_sequential_fp8(const void* base_logits, const void* w1, const uint8_t* w2q,
                                 const uint16_t* w2_scales, const int64_t* prev,
                                 const int64_t* seeds, const int64_t* positions, int32_t k,
                                 const float* temperature, void* cache, int64_t* tokens,
                                 markov_stream_t stream, const markov_shape_t* shape,
                                 void* workspace, size_t workspace_bytes);

/* markov_greedy_sequential with the E4M3 w2 (the page's
 * `dsparkMarkovGreedyFusedStepFp8`); arguments as the two above. */
int markov_greedy_sequential_fp8(const void* base_logits, const void* w1, const uint8_t* w2q,
                                 const uint16_t* w2_scales, const int64_t* prev, int32_t k,
                                 void* cache, int64_t* tokens, uint64_t* winners,
                                 markov_stream_t stream, const markov_shape_t* shape,
                                 void* workspace, size_t workspace_bytes);

/* One step of either E4M3 loop alone (as markov_sample_step and
 * markov_greedy_step are to their loops). */
int markov_sample_step_fp8(const void* base_logits, const void* w1, const uint8_t* w2q,
                           const uint16_t* w2_scales, const int64_t* prev, const int64_t* seeds,
                           const int64_t* positions, int32_t k, int32_t step,
                           const float* temperature, void* cache, int64_t* tokens,
                           markov_stream_t stream, const markov_shape_t* shape, void* workspace,
                           size_t workspace_bytes);
int markov_greedy_step_fp8(const void* base_logits, const void* w1, const uint8_t* w2q,
                           const uint16_t* w2_scales, const int64_t* prev, int32_t k, int32_t step,
                           void* cache, int64_t* tokens, uint64_t* winners, markov_stream_t stream,
                           const markov_shape_t* shape, void* workspace, size_t workspace_bytes);

/* ---- one GPU's share of a vocabulary-parallel step (vLLM muse_spark
 * cutedsl draft Markov page: module docstring on tensor-parallel drafting,
 * the last block's packet, `_PickKernel` / `markov_pick`) -------------------- */

/*
 * One draft step on the vocabulary slab [vocab_offset, vocab_offset + V) of
 * a vocabulary of vocab_total tokens, where V = shape->vocab (a multiple of
 * 8): the same arithmetic as markov_sample_sequential's step `step`, with
 * every token id global (the noise hash and the packed winner use
 * vocab_offset + local id), so that the shards' winners combine into the
 * full-vocabulary token.
 *   base_logits, cache  device bf16 [rows, k, V]: this slab's columns
 *   w1                  device bf16 [vocab_total, R]: every row (any token feeds)
 *   w2                  device bf16 [V, R]: this slab's rows
 *   feed                device int64, row r's feeding token at feed[r *
 *                       feed_stride] (global id; clamped as unsigned to
 *                       vocab_total - 1), e.g. the picked tokens of step-1
 *   seeds, positions, k, step, temperature  as markov_sample_sequential
 *   packets             device uint64 [rows] (write): the slab's winner of
 *                       each row, packed as markov_greedy_sequential's winners
 *                       (an orderable key of the winning noised logit, then
 *                       the complement of its global id)
 *   workspace           as markov_sample_sequential, for this shape
 * One kernel launch; the workgroup that finishes last writes the packets and
 * re-zeroes the workspace's slots. Errors: as markov_sample_sequential, and
 * MARKOV_ERR_SHAPE for step outside [0, k), feed_stride < 1, or a slab
 * outside [0, vocab_total), MARKOV_ERR_VOCAB for vocab_total above
 * MARKOV_MAX_VOCAB.
 */
int markov_shard_step(const void* base_logits, const void* w1, const void* w2, const int64_t* feed,
                      int64_t feed_stride, const int64_t* seeds, const int64_t* positions,
                      int32_t k, int32_t step, const float* temperature, void* cache,
                      uint64_t* packets, int32_t vocab_offset, int32_t vocab_total,
                      markov_stream_t stream, const markov_shape_t* shape, void* workspace,
                      size_t workspace_bytes);

/*
 * The token of each row over `shards` slabs' packets (device uint64
 * [shards, rows], e.g. gathered from every GPU): the largest packet, so the
 * first NaN key, else the largest key, else the lowest global id.
 * tokens[r * stride] gets the global id (device int64; stride >= 1, e.g. k to
 * fill column s of a [rows, k] array), and winner[r] (device uint64, or
 * NULL) the winning packet. One small kernel on `stream`.
 */
int markov_pick(const uint64_t* packets, int32_t shards, int32_t rows, int64_t* tokens,
                int64_t stride, uint64_t* winner, markov_stream_t stream);

/* ---- verification of a drafted block (TensorRT Edge-LLM "DSpark kernels"
 * page: `dsparkGreedyAccept`, `dsparkProbabilisticAccept`) --------------------
 *
 * Shapes: B rows, P proposals per row, V tokens. Draft token j of row b
 * (draft[b * draft_stride + j], j < P) sits at verify position j + 1 and is
 * checked against the target at position j. proposal_lengths[b] = L_b (int32;
 * above P counts as P, below 0 as 0). Outputs: accepted int64 [B, P + 1],
 * the accepted drafts then one more token, -1 after; accept_len int32 [B],
 * their count (accepted drafts + 1). workspace: device, at least
 * markov_verify_workspace_bytes(B, P), 16-byte aligned, zeroed once by the
 * caller (hipMemset) and left zeroed by every call; not shared by two calls
 * in flight. One kernel launch each, no host synchronisation. Errors:
 * MARKOV_ERR_SHAPE (B < 1, P < 0, draft_stride < P, V out of range),
 * MARKOV_ERR_VOCAB (V above MARKOV_MAX_VOCAB), MARKOV_ERR_NULL,
 * MARKOV_ERR_ALIGN, MARKOV_ERR_WORKSPACE, MARKOV_ERR_HIP.
 */
size_t markov_verify_workspace_bytes(int32_t batch, int32_t proposal_len);

/*
 * Greedy: a_j = the first NaN, else the lowest id of the largest value of
 * target_logits[b][j][0..V) (device bf16 [B, P+1, V], 16-byte aligned, V a
 * multiple of 8). Drafts j = 0, 1, ... are accepted while draft j == a_j and
 * j < L_b; the token after them is a_n (n accepted), the base's bonus token.
 */
int markov_greedy_accept(const void* target_logits, const int64_t* draft, int32_t draft_stride,
                         const int32_t* proposal_lengths, int64_t* accepted, int32_t* accept_len,
                         int32_t batch, int32_t proposal_len, int32_t vocab, void* workspace,
                         size_t workspace_bytes, markov_stream_t stream);

/*
 * Probabilistic (speculative sampling with a residual): target_probs p
 * device fp32 [B, P+1, V], draft_probs q device fp32 [B, P, V], uniforms
 * device fp32 [B, 2P+1]. Draft j (token d) is accepted iff u_j q_j(d) <
 * p_j(d), both products exact in binary64 (an id outside [0, V) never is).
 * At the first rejection j the token after the accepted drafts is sampled
 * from r(x) = max(0, RN32(p_j(x) - q_j(x))) with u_{P+j}; if all L_b drafts
 * pass, from p_{L_b} with u_{2P}. Sampling with u from weights w: the
 * smallest x whose running sum of w exceeds u times the total, sums in
 * binary64 (their order is the kernel's own, so the token may differ from
 * an index-order sum only where u times the total lies within a few
 * binary64 ulps of a running sum); with no residual mass p_j itself is
 * sampled, and with none either token 0.
 */
int markov_prob_accept(const float* target_probs, const float* draft_probs, const int64_t* draft,
                       int32_t draft_stride, const int32_t* proposal_lengths, const float* uniforms,
                       int64_t* accepted, int32_t* accept_len, int32_t batch, int32_t proposal_len,
                       int32_t vocab, void* workspace, size_t workspace_bytes,
                       markov_stream_t stream);

/* A readable name of a status code (static string). */
const char* markov_status_string(int status);

/* ---- test-only entry points ------------------------------------------- */

/* markov_sample_sequential with the exact key taken at every element (no
 * pruning by the cheap key estimate); the tokens must be the same. */
int markov_debug_sample_fallback(const void* base_logits, const void* w1, const void* w2,
                                 const int64_t* prev, const int64_t* seeds,
                                 const int64_t* positions, int32_t k, const float* temperature,
                                 void* cache, int64_t* tokens, markov_stream_t stream,
                                 const markov_shape_t* shape, void* workspace,
                                 size_t workspace_bytes);
/* (markov_debug_sample_fallback above: every noisy row of every workgroup
 * takes the exact re-read path that near-ties and non-finite estimates
 * take; the tokens must be the same.) */
int markov_debug_sample_exact(const void* base_logits, const void* w1, const void* w2,
                              const int64_t* prev, const int64_t* seeds,
                              const int64_t* positions, int32_t k, const float* temperature,
                              void* cache, int64_t* tokens, markov_stream_t stream,
                              const markov_shape_t* shape, void* workspace,
                              size_t workspace_bytes);

/*
 * The bias alone, through the step kernel's own contraction path:
 * bias[r][v] = bf16(sum_j w1[min_u64(tok[r], V-1)][j] * w2[v][j]).
 *   w1, w2 device bf16 [V, R]; tok device int64 [rows]; bias device bf16
 *   [rows, V] (write). Same error rules as markov_sample_sequential.
 */
int markov_debug_bias(const void* w1, const void* w2, const int64_t* tok, void* bias,
                      const markov_shape_t* shape, markov_stream_t stream);

/*
 * The Gumbel key of n (logit, token id) pairs of one row at one step:
 * key_exact is the key the kernel's argmax uses; key_upper is the kernel's
 * cheap upper bound of it (the noise bound table lookup plus the logit term),
 * key_exact <= key_upper for every input with a finite bound. `workspace` is
 * a workspace prepared by markov_workspace_init (it holds the table). All
 * arrays device, length n; logits fp32, ids uint32, outputs fp32.
 */
int markov_debug_gumbel(const float* logits, const uint32_t* ids, int64_t n, float temperature,
                        int64_t seed, int32_t step, int64_t position, const void* workspace,
                        float* key_exact, float* key_upper, markov_stream_t stream);

/* RN bf16 of n binary32 values with the kernel's conversion (test-only). */
int markov_debug_bf16_round(const float* in, uint16_t* out, int64_t n, markov_stream_t stream);

/* The noise bound tables, host side (test-only): for the first n of the
 * 2050 hash buckets, three binary32 values each into out[3 n] (host
 * memory): the bucket line's A and B (the kernel bounds the noise of a hash
 * h of the bucket by fma(B, float(h), A)) and the constant bound C (the
 * bucket's largest noise plus 1e-5). Returns the number of buckets written. */
int32_t markov_debug_noise_table(float* out, int32_t n);

/* The output-transform table, host side (test-only): the first n (at most
 * 32768) entries of the table markov_workspace_init stamps for this mult and
 * softcap (softcap > 0), bf16 bit patterns into out[n] (host memory).
 * Returns the number of entries written. */
int32_t markov_debug_transform_table(float mult, float softcap, uint16_t* out, int32_t n);

/* The E4M3 code of each of n binary32 values with the quantizer's own
 * rounding (test-only; device arrays). */
int markov_debug_e4m3_encode(const float* x, uint8_t* out, int64_t n, markov_stream_t stream);

/* The bf16 values of n E4M3 codes (n a multiple of 8; codes 8-byte aligned,
 * out 16-byte aligned) through the step kernel's own decode (test-only). */
int markov_debug_e4m3_decode(const uint8_t* codes, void* out, int64_t n, markov_stream_t stream);

/* markov_debug_bias with the E4M3 w2 (test-only). */
int markov_debug_bias_fp8(const void* w1, const uint8_t* w2q, const uint16_t* w2_scales,
                          const int64_t* tok, void* bias, const markov_shape_t* shape,
                          markov_stream_t stream);

/* A plain device copy of `bytes` (a multiple of 16; both pointers 16-byte
 * aligned) from src to dst on `stream` (test-only): the reference kernel
 * whose counter readings calibrate DRAM byte counts. */
int markov_debug_copy(const void* src, void* dst, int64_t bytes, markov_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MARKOV_H_ */
