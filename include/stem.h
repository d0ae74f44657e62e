/*
 * stem.h - C ABI of the MI355X (gfx950) Stem sparse-prefill attention library.
 *
 * The path has three stages, each one entry point:
 *   stem_score          block-level scoring: stride-s anti-diagonal down-sampled
 *                       Q.K^T, max-pooled to block x block scores, plus the
 *                       output-aware value bonus (stem_score_fp8: the same on
 *                       e4m3 codes with per-block scales).
 *   stem_schedule_topk  Token-Position-Decay budget per query block, sink and
 *                       window blocks forced, per-row top-k -> compact lists.
 *   stem_bsa_prefill    causal block-sparse flash attention over those lists
 *                       (bf16, or fp8 e4m3 with per-block scales, with e4m3 or
 *                       fp16 attention weights for P.V).
 * plus stem_dense_prefill, the library's own dense causal attention (the
 * baseline every speed-up is measured against), and two variants of stage 3:
 * stem_bsa_prefill_paged (fp8 K/V in a page pool addressed by a block table)
 * and stem_bsa_prefill_q64 (lists over 64-query rows against 128-key blocks).
 *
 * Sources: AngelSlim documentation "Stem: Rethinking Causal Information Flow in
 * Sparse Attention" §2.1-2.3 and the §6 parameter table; gist.science summary of the Stem paper, §2.1 (TPD budget)
 * and §2.2 (OAM metric).
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE memory owned by the caller; the library keeps
 *    no pointer after the call returns and allocates nothing.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  The host never waits for the device.  Every call
 *    enqueues kernel launches only (no memset, copy or allocation), so a
 *    sequence of calls can be captured into a HIP graph and replayed; launch
 *    arguments (shapes, k_start, the softmax scale, ...) are fixed at capture.
 *  - Arguments are validated before anything is enqueued; an invalid call
 *    returns a non-zero stem_status_t and enqueues nothing.  A launch failure
 *    returns STEM_ERR_HIP.  Device-side faults surface at the caller's next
 *    synchronisation on that stream.
 *  - Calls on different streams are independent; the library holds no state
 *    and is thread-safe.
 *  - Token-major layouts: Q is [T][Hq][d], K and V are [T][Hkv][d] (row
 *    stride H*d elements), T = total packed tokens.  Sequences are packed back
 *    to back; cu_seqlens holds the num_seqs+1 token offsets.  Query head h
 *    reads KV head h / (Hq / Hkv) (grouped-query attention).
 *  - Blocks are counted per sequence: sequence z has nb_z = L_z / block_size
 *    blocks, and query-block rows are numbered globally r = 0 .. R-1 with
 *    R = sum_z nb_z (key blocks use the same global numbering).  max_nb =
 *    max_z nb_z.
 */
#ifndef STEM_H_
#define STEM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STEM_OK = 0,
  STEM_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent shape  */
  STEM_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head_dim != 128,
                                 block_size != 128, ragged tail block, ...)  */
  STEM_ERR_CAPACITY = 3,      /* k_cap smaller than a row's kept count       */
  STEM_ERR_WORKSPACE = 4,     /* workspace missing or too small              */
  STEM_ERR_HIP = 5            /* a HIP launch or runtime call failed         */
} stem_status_t;

typedef enum {
  STEM_DTYPE_BF16 = 0,        /* bfloat16 Q/K/V                              */
  STEM_DTYPE_FP8_E4M3 = 1,    /* OCP e4m3fn codes with fp32 per-block scales  */
  STEM_DTYPE_FP8_E4M3_PV16 = 2 /* the same inputs; P.V with fp16 weights     */
} stem_dtype_t;

/* One packed batch of sequences (the shape of the problem). */
typedef struct {
  int32_t num_seqs;                 /* B >= 1                                   */
  const int32_t *cu_seqlens_host;   /* HOST [B+1]: 0 = c0 < c1 < ..., every
                                       length c[z+1]-c[z] a positive multiple of
                                       block_size.  Read during the call only;
                                       the kernels receive the offsets by value */
  int32_t num_q_heads;              /* Hq, a multiple of num_kv_heads           */
  int32_t num_kv_heads;             /* Hkv >= 1                                 */
  int32_t head_dim;                 /* d; 128 is the supported value            */
  int32_t block_size;               /* attention block; 128 is supported        */
} stem_problem_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char *stem_status_string(int status);

/* ---------------------------------------------------------------------------
 * Stage 1: block scores.  AngelSlim Stem doc §2.1: score(Q_i, K_j) =
 * Q_i.K_j^T / (sqrt(d) s n) + lambda ReLU(vbar_j), computed by a strided
 * group GEMM with stride s and chunk width chunk_size; gist.science summary
 * §2.2-2.3: anti-diagonal down-sampling of Q and K, block-wise max pooling,
 * value magnitude from block max pooling.
 *
 * For sequence z, query head h, KV head g, strided rows i, j in [0, L_z/s):
 *   A[i][j] = sum_{t<s} Q[c_z + i s + t][h] . K[c_z + j s + s-1-t][g]
 *             / (sqrt(d) * s * norm),     defined for j <= i
 *   S[h][r(z,I)][J] = max over the (block/s)^2 strided cells of block pair
 *                     (I, J) with j <= i, plus bonus[g][J], for J <= I
 *   bonus[g][J] = beta * max(0, (l_J - mean_z(l)) / (std_z(l) + 1e-6)),
 *   l_J = ln max_{t in key block J} ||V[t][g]||^2, mean and population std
 *   taken over the nb_z key blocks of sequence z.
 * S is fp32 [Hq][R][max_nb]; every entry with J > I or J >= nb_z is -inf.
 * q, k, v: bf16.  stride must divide block_size (else INVALID_ARG); stride 8
 * is the one implemented (others return UNSUPPORTED).  chunk_size is a
 * positive multiple of block_size (it orders the work, it changes no value).
 * Sequences of more than 65536 blocks (8M tokens) return UNSUPPORTED.
 * workspace: device memory of at least stem_score_workspace_bytes(p) bytes
 * (one fp32 per KV head and key block, then 32 bytes of work-queue counters
 * per 64 sequences, each part rounded up to 256 bytes), 256-byte aligned; its
 * contents on return are unspecified.
 * ------------------------------------------------------------------------- */
size_t stem_score_workspace_bytes(const stem_problem_t *p);
int stem_score(const stem_problem_t *p, const void *q, const void *k, const void *v,
               int32_t stride, int32_t chunk_size, float norm, float beta,
               float *scores, void *workspace, size_t workspace_bytes, void *stream);

/* stem_score for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation and result as stem_score, with the library's own device
 * array of STEM_SCORE_SCRATCH_BYTES (1 MiB + 4 KiB, one per GPU, held until
 * the process ends) in place of the workspace argument: it serves every
 * problem whose stem_score_workspace_bytes fits, which includes all with
 * num_kv_heads * R <= 262144 (e.g. 8 KV heads and 4M tokens) and at most
 * 8192 sequences.  Larger problems return STEM_ERR_WORKSPACE before
 * anything is enqueued.  The call
 * allocates nothing; its first call on a GPU (the device of `stream`, or the
 * current device for the null stream) looks up that GPU's array address
 * (hipGetSymbolAddress), so a caller that will capture should make one call
 * on that device beforehand.  Every call on a GPU uses that GPU's one array:
 * calls that overlap on one GPU (different streams, threads or graphs in
 * flight together) race and must be serialised by the caller.  The array's
 * contents are rewritten by every call before they are read. */
#define STEM_SCORE_SCRATCH_BYTES ((1u << 20) + 4096u)
int stem_score_noalloc(const stem_problem_t *p, const void *q, const void *k, const void *v,
                       int32_t stride, int32_t chunk_size, float norm, float beta,
                       float *scores, void *stream);

/* Stage 1 on e4m3 inputs: the scores above, with Q, K and V the dequantised
 * values code * scale (the e4m3 layout of stem_bsa_prefill: codes [T][H][d],
 * fp32 scales [R][H] per (128-token block, head), all device memory).  The
 * strided products run on the fp8 matrix cores; each block pair's pooled
 * maximum is multiplied by its query and key block scales, which are constant
 * over the pair's strided cells, and the value bonus uses
 * ||V_t||^2 = v_scale^2 sum_d code_d^2.  The fp8 MFMA sums its 64 products
 * per step to about 2^-15 of their absolute sum (not fp32 rounding): on
 * unit-variance inputs the scores stay within 3e-5 of max(|score|, 1) of the
 * exact scores of the dequantised values.  A null scale pointer returns
 * INVALID_ARG; everything else as stem_score (same workspace size). */
int stem_score_fp8(const stem_problem_t *p, const void *q, const void *k, const void *v,
                   const float *q_scale, const float *k_scale, const float *v_scale,
                   int32_t stride, int32_t chunk_size, float norm, float beta,
                   float *scores, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Stage 2: schedule + top-k.  gist.science summary §2.1 (TPD): per query
 * block I of a sequence with nb blocks, k(I) = floor(ke - ke (1-mu) I / nb),
 * ke = alpha * k_start (alpha: this layer's factor, AngelSlim doc §2.2);
 * AngelSlim doc §2.2 / zhichai summary §三: the first n_init blocks (sinks)
 * and the n_window blocks ending at I are always kept.
 *   F(I)     = [0, min(n_init, I+1)) U [max(0, I-n_window+1), I]
 *   kept(I)  = min(I+1, max(k(I), |F(I)|))
 * Row (h, r) lists F(I) plus the kept(I)-|F(I)| best other blocks J <= I by
 * score (descending; equal scores -> lower J first; NaN ranks as -inf),
 * in ascending order.  block_idx: int32 [Hq][R][k_cap], entries past the
 * count are -1; block_cnt: int32 [Hq][R].
 * k_start_host: HOST [B] budgets in blocks (before alpha), >= 0.
 * mu in (0, 1], alpha > 0, n_init >= 0, n_window >= 0.
 * k(I) is evaluated in fp64 as floor(x + 1e-9): exact whenever the
 * parameters' decimal values have denominators far below 1e9 (e.g. 0.7 =
 * 7/10), which every documented setting has.
 * Returns STEM_ERR_CAPACITY if k_cap < stem_max_kept(...).  Requires
 * max_nb <= 2048 (sequences up to 256K tokens at block 128).
 * ------------------------------------------------------------------------- */
int stem_schedule_topk(const stem_problem_t *p, const float *scores,
                       const double *k_start_host, double mu, double alpha,
                       int32_t n_init, int32_t n_window, int32_t k_cap,
                       int32_t *block_idx, int32_t *block_cnt, void *stream);

/* Host-only helpers (no device work): the budget rule above, and the
 * largest kept(I) over every row of the problem (a safe k_cap). */
int32_t stem_tpd_budget(int32_t I, int32_t nb, double k_start, double mu, double alpha);
int32_t stem_kept_count(int32_t I, int32_t nb, double k_start, double mu, double alpha,
                        int32_t n_init, int32_t n_window);
int32_t stem_max_kept(const stem_problem_t *p, const double *k_start_host, double mu,
                      double alpha, int32_t n_init, int32_t n_window);

/* ---------------------------------------------------------------------------
 * Workspace of stem_bsa_prefill / stem_dense_prefill: device memory of at
 * least this many bytes, 256-byte aligned (0 for an invalid problem or
 * dtype).  Each call first rewrites it with V in the tile layout the
 * attention kernel loads (per KV head and key block, the 128 x 128 V^T tile
 * with one 16-byte pad chunk per row; fp16 for bf16 inputs, e4m3 for fp8
 * inputs, plus fp16 for FP8_E4M3_PV16): T * Hkv * 272 bytes for bf16; for
 * fp8 (either dtype), T * Hkv * 416
 * bytes plus 8 bytes per (key block, KV head) for the row-indexed K and V
 * scales that stem_bsa_prefill_paged gathers from its pages (d = 128);
 * rounded up to 256 bytes, then the work queues of the attention kernel:
 * 32 bytes per launch of up to 64 sequences, rounded up to 256 bytes.
 * Contents on return are unspecified; concurrent calls need separate
 * workspaces.
 * ------------------------------------------------------------------------- */
size_t stem_attn_workspace_bytes(const stem_problem_t *p, int32_t dtype);   /* FP8_E4M3_PV16: as fp8 */

/* ---------------------------------------------------------------------------
 * Stage 3: causal block-sparse attention.  AngelSlim doc §2.3: exact
 * attention on the selected blocks only; youleyou HPC-BSA article §三.3.1: a
 * skipped block is equivalent to all its scores being -inf.
 * For row (h, r) = (h, block I of sequence z), queries t in block I attend to
 * the keys of the listed blocks J (local to z) with key position <= query
 * position: out[t][h] = sum_u softmax_u(softmax_scale * q_t.k_u) v_u.
 * A row with count 0 gives out = 0 and lse = -inf.
 * dtype BF16: q, k, v bf16; scales must be NULL.
 * dtype FP8_E4M3: q, k, v are e4m3fn codes (uint8); the real value of an
 *   element of token block b (global) and head x is code * scale[b][x]:
 *   q_scale fp32 [R][Hq], k_scale and v_scale fp32 [R][Hkv].  Scales are
 *   finite and >= 0 (an amax / 448 quantiser gives that); a zero scale is a
 *   block of zeros whatever its codes (its keys keep their softmax share and
 *   add nothing to the output).  Negative or non-finite scales are outside
 *   the contract: the device cannot report them, and the output is then
 *   unspecified (no memory is accessed out of bounds).
 * block_idx / block_cnt as produced by stem_schedule_topk (k_cap = its row
 *   stride; entries must be ascending, in [0, I]).
 * out: bf16 [T][Hq][d].  lse: optional fp32 [Hq][T] (natural log), may be NULL.
 * workspace: see stem_attn_workspace_bytes (STEM_ERR_WORKSPACE if too small).
 * Precision: Q.K^T in the input type (bf16, or e4m3 with fp32 scales), fp32
 * accumulation and softmax; P.V with P rounded to fp16 against an exact fp16
 * copy of V for bf16 inputs (V magnitudes above 65504 saturate to +-65504:
 * such inputs are outside the bf16 contract), and to e4m3 for fp8 inputs
 * (each weight times the block's V scale, relative to a running reference
 * that keeps the largest weight between 152 and 430, below e4m3's 448).
 * An e4m3 weight is off by up to 2^-4 of itself; that averages out over many
 * keys of similar weight but not when a few keys hold a query's attention, so
 * for every 32 queries a half block (64 keys) in which some query's largest
 * weight exceeds 1/8 of that query's weight sum so far, and the diagonal
 * block, get a second e4m3 P.V pass with the rounding residuals (about 2^-8
 * per weight in all).  On the synthetic workloads and on
 * concentrated attention (logits scaled up to 8x) the fp8 output stays within
 * max-abs 6e-2 of exact attention on the dequantised inputs.
 * ------------------------------------------------------------------------- */
int stem_bsa_prefill(const stem_problem_t *p, int32_t dtype, const void *q, const void *k,
                     const void *v, const float *q_scale, const float *k_scale,
                     const float *v_scale, const int32_t *block_idx,
                     const int32_t *block_cnt, int32_t k_cap, float softmax_scale,
                     void *out, float *lse, void *workspace, size_t workspace_bytes,
                     void *stream);

/* dtype FP8_E4M3_PV16 takes the FP8_E4M3 inputs and scales but runs every
 * block's P.V with fp16 weights against an exact fp16 V^T image.  The e4m3 weight rounding (relative error up to 2^-4 per weight)
 * averages out when attention is spread over many keys, but not when a few
 * keys hold it; this dtype keeps such rows at bf16-level output error, for
 * about 1.35x the e4m3 time.  Q.K^T stays e4m3 in both: the fp8 MFMA sums its
 * 64 products per step with less than fp32 precision (measured error up to
 * 2^-15 of the sum of |products| on quantised Gaussian data), which shows in
 * the LSE of very large logits.  Taken by stem_bsa_prefill and
 * stem_dense_prefill (the paged and 64-query entry points have no dtype
 * argument and no such mode).
 * ------------------------------------------------------------------------- */

/* ---------------------------------------------------------------------------
 * Dense causal attention with the same tile kernel (every causal block): the
 * baseline of the AngelSlim doc §2.3 (its bf16 dense prefill, next to the
 * fp8 block-sparse one) and of the §3 support table's dense entries; every
 * speed-up of the sparse path is measured against it.
 * out[t][h] = sum_{u <= t} softmax_u(softmax_scale * q_t.k_u) v_u per
 * sequence (keys of earlier sequences never attend).  Same arguments, layout,
 * precision and errors as stem_bsa_prefill without the lists; equal to
 * stem_bsa_prefill with every causal block listed, bit for bit.
 * ------------------------------------------------------------------------- */
int stem_dense_prefill(const stem_problem_t *p, int32_t dtype, const void *q, const void *k,
                       const void *v, const float *q_scale, const float *k_scale,
                       const float *v_scale, float softmax_scale, void *out, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Block-sparse attention on a paged fp8 K/V cache (the AngelSlim doc's
 * "paged" fp8 execution path, §6 parameter table: hpc_fp8_path; §3 support
 * table).  The pages name the path but not its layout; this reading keeps
 * everything as in stem_bsa_prefill with STEM_DTYPE_FP8_E4M3 except where K
 * and V live:
 * q, q_scale: as stem_bsa_prefill (packed varlen e4m3 [T][Hq][d], fp32 [R][Hq]).
 * k_pages, v_pages: e4m3 pools of num_pages pages of block_size tokens,
 *   [page][token][Hkv][d] (one page per 128-token key block).
 * k_scale_pages, v_scale_pages: fp32 [num_pages][Hkv], per page and KV head.
 * block_table: device int32 [num_seqs][table_stride]; entry [z][J] is the
 *   page holding key block J of sequence z, for J < nb_z.  Entries outside
 *   [0, num_pages) are clamped into it (never read out of the pool).
 * block_idx, block_cnt, k_cap, softmax_scale, out, lse, workspace: as
 *   stem_bsa_prefill (workspace: stem_attn_workspace_bytes(p, FP8)).
 * Errors: INVALID_ARG for a null table, num_pages < 1 or table_stride below
 *   the longest sequence's block count, plus those of stem_bsa_prefill.
 * The result equals stem_bsa_prefill on the same blocks laid out contiguously.
 * ------------------------------------------------------------------------- */
int stem_bsa_prefill_paged(const stem_problem_t *p, const void *q, const void *k_pages,
                           const void *v_pages, const float *q_scale, const float *k_scale_pages,
                           const float *v_scale_pages, const int32_t *block_table,
                           int32_t table_stride, int32_t num_pages, const int32_t *block_idx,
                           const int32_t *block_cnt, int32_t k_cap, float softmax_scale, void *out,
                           float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Block-sparse attention with 64-query rows against 128-key blocks (bf16).
 * The youleyou HPC-BSA article §三.3.1 names 64 x 128 blocks next to
 * 128 x 128; this entry point takes lists over query blocks of 64 tokens:
 * list row 2 r + s (s = 0, 1) covers queries [64 s, 64 s + 64) of block row
 * r (r as in stem_bsa_prefill), and its entries are 128-token key-block ids
 * J (local to the sequence), ascending, in [0, I] with I the row's block
 * index; keys later than the query are masked as in stem_bsa_prefill.
 * block_idx: int32 [Hq][2 R][k_cap]; block_cnt: int32 [Hq][2 R].
 * q, k, v: bf16 as in stem_bsa_prefill; out, lse, softmax_scale, workspace
 *   (stem_attn_workspace_bytes(p, BF16)) likewise.  Precision as the bf16
 *   path of stem_bsa_prefill.
 * Giving both halves of a row the row's list reproduces stem_bsa_prefill
 * bit for bit.  The kernel walks the union of the two lists with the row's
 * 128 queries; the waves of a half skip the MFMAs and the softmax of a block
 * their half does not list, so the cost follows the per-half work plus a
 * share of the union (about 1.4x the square-row call per computed pair on
 * independent half lists at 25 %, 1.1x on identical ones).
 * Errors: as stem_bsa_prefill with dtype BF16; UNSUPPORTED for a sequence
 * longer than 4096 key blocks (512K tokens).
 * ------------------------------------------------------------------------- */
int stem_bsa_prefill_q64(const stem_problem_t *p, const void *q, const void *k, const void *v,
                         const int32_t *block_idx, const int32_t *block_cnt, int32_t k_cap,
                         float softmax_scale, void *out, float *lse, void *workspace,
                         size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* STEM_H_ */
