// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
// Nothing here is part of the public ABI (include/stem.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace stem {

constexpr int kBlock = 128;           // attention block (tokens)
constexpr int kHeadDim = 128;         // head dimension
constexpr int kMaxSeqsPerLaunch = 64; // sequences described inline per launch
constexpr int kMaxRowBlocks = 2048;   // top-k row length limit (256K tokens)
constexpr int kMaxListBlocks = 4096;  // 64-query-row attention: longest sequence (key blocks)
constexpr int kMaxScoreBlocks = 65536; // scoring: longest sequence (key blocks; 32-bit tile indexing)

// Packed-batch description passed BY VALUE to every kernel (no device
// metadata buffers).  Offsets are global: tok[z] is the first packed token of
// sequence z of this launch, row[z] its first global block row (tok[z]/128).
// item[z] is a per-kernel prefix of work items (set by the launcher).
struct SeqTable {
  int32_t n;
  int32_t z0;                       // global index of the launch's first sequence
  int32_t tok[kMaxSeqsPerLaunch + 1];
  int32_t row[kMaxSeqsPerLaunch + 1];
  int32_t item[kMaxSeqsPerLaunch + 1];
};

// Locate the sequence of this launch that contains `x`, where `off` is a
// non-decreasing prefix array of n+1 entries (row offsets or item offsets).
__device__ __forceinline__ int seq_of(const int32_t *off, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {               // largest z with off[z] <= x
    int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Work-item order for a grid whose hardware dispatch sends workgroup b to
// XCD b % 8 (MI355X: 8 XCDs, each with its own L2).  Items are "slots"
// (a row or tile of one KV group) times G query heads.  In every round of
// 8*G consecutive workgroups, the 8 XCDs take 8 consecutive slots and each
// XCD runs all G heads of its slot, so the heads that share K/V meet in one
// L2 and the whole chip walks the same KV head at the same time.
// Returns slot * G + head.
__device__ __forceinline__ int xcd_item(int b, int n_items, int G) {
  const int per_round = 8 * G;
  const int full = (n_items / per_round) * per_round;
  if (b >= full) return b;                       // ragged last round: identity
  const int round = b / per_round, j = b - round * per_round;
  const int slot = round * 8 + (j & 7);
  return slot * G + (j >> 3);
}

// Work-item order that gives each XCD a contiguous eighth of the items:
// workgroup b runs on XCD b % 8 as the (b / 8)-th workgroup that XCD
// receives, so XCD x walks items [x n/8, (x+1) n/8) in order.  With items
// ordered KV group first, then rows, then the G heads of a row, each XCD
// (own L2) keeps neighbouring rows of one KV group in flight, and those
// rows' heads list mostly the same K/V blocks.  A ragged tail (n not a
// multiple of 8) keeps the identity order.
__device__ __forceinline__ int xcd_chunk_item(int b, int n_items) {
  const int per = n_items >> 3;
  if (b >= per * 8) return b;
  return (b & 7) * per + (b >> 3);
}

// Token-Position-Decay budget: k(I) = floor(ke - ke (1 - mu) I / nb), with
// ke = alpha * k_start already folded in.  Evaluated in fp64 without
// contraction; the 1e-9 nudge absorbs the rounding of the fp64 steps when the
// exact (decimal) value is an integer.
__host__ __device__ inline int tpd_budget(int I, int nb, double ke, double mu) {
#pragma clang fp contract(off)
  const double slope = ke * (1.0 - mu);
  const double dec = slope * (double)I / (double)nb;
  const double x = ke - dec;
  return (int)floor(x + 1e-9);
}

__host__ __device__ inline int forced_count(int I, int n_init, int n_window) {
  // |[0, min(n_init, I+1)) U [max(0, I-n_window+1), I]|
  const int a = n_init < I + 1 ? n_init : I + 1;          // sinks [0, a)
  int w0 = I - n_window + 1; if (w0 < 0) w0 = 0;         // window [w0, I]
  const int wn = n_window > 0 ? I - w0 + 1 : 0;
  if (wn == 0) return a;
  const int overlap = a > w0 ? a - w0 : 0;
  return a + wn - overlap;
}

__host__ __device__ inline int kept_count(int I, int nb, double ke, double mu,
                                          int n_init, int n_window) {
  int k = tpd_budget(I, nb, ke, mu);
  const int f = forced_count(I, n_init, n_window);
  if (k < f) k = f;
  return k < I + 1 ? k : I + 1;
}

// Score tiles of one (sequence, query head) with nb blocks: the causal
// triangle of 256 x 256 strided tiles (16 x 16 blocks each).
__host__ __device__ inline int score_pairs(int nb) {
  const int nt = (nb + 15) / 16;
  return nt * (nt + 1) / 2;
}

// ---------------------------------------------------------------- launchers
struct ScoreLaunch {
  const void *q, *k, *v;
  const float *q_scale, *k_scale, *v_scale;   // e4m3 inputs: per (block, head); else null
  float *scores, *ell;          // ell: workspace [Hkv][R] (log norms, then bonus)
  int32_t *ctr;                 // workspace: 8 work-queue counters per score launch
  int32_t n_ctr;
  int32_t Hq, Hkv, R, max_nb;
  int32_t stride, chunk_size;
  float scale, beta;
  bool fp8;
};
hipError_t launch_vnorm(const ScoreLaunch &a, hipStream_t s);
hipError_t launch_vstats(const ScoreLaunch &a, const SeqTable &t, hipStream_t s);
hipError_t launch_score(const ScoreLaunch &a, const SeqTable &t, int n_items, int launch_index, hipStream_t s);
// Score workspace: ell [Hkv][R] fp32, then the counters, each part 256-byte aligned.
size_t score_workspace_ctr_offset(int Hkv, int R);
size_t score_workspace_bytes(int Hkv, int R, int num_seqs);

struct TopkLaunch {
  const float *scores;
  int32_t *idx, *cnt;
  int32_t Hq, R, max_nb, k_cap;
  double mu;
  int32_t n_init, n_window;
  double ke[kMaxSeqsPerLaunch];
};
hipError_t launch_topk(const TopkLaunch &a, const SeqTable &t, int rows_in_launch, hipStream_t s);

struct AttnLaunch {
  const void *q, *k, *v;
  const float *q_scale, *k_scale, *v_scale;
  const int32_t *idx, *cnt;
  int32_t k_cap;
  void *out;
  float *lse;
  uint16_t *vimg16;              // workspace: fp16 V^T tile images [Hkv][R][128 rows x 136]
  uint8_t *vimg8;                // workspace (fp8 only): e4m3 V^T tile images [Hkv][R][128 x 144 B]
  int32_t Hq, Hkv, R, T;
  float scale_log2;              // softmax_scale * log2(e)
  // Paged K/V (fp8 only; null table = contiguous varlen tensors): k and v
  // point at pools of num_pages pages of kBlock tokens, [page][token][Hkv][d];
  // table[z * table_stride + J] is the page of key block J of sequence z;
  // the caller's scales k_scale_pages / v_scale_pages are [page][Hkv], and
  // k_scale / v_scale then point at row-indexed copies in the workspace
  // that the paged pre-pass fills.
  const int32_t *table;
  int32_t table_stride, num_pages;
  const float *k_scale_pages, *v_scale_pages;
  // Work queues of the persistent bf16 kernel: 8 counters (one per XCD) per
  // launch, in the workspace; the V^T pre-pass zeroes n_ctr of them.
  int32_t *ctr;
  int32_t n_ctr;
};
// fp8 workspace: e4m3 V^T images, then fp16 ones, then K and V scales [R][Hkv]
// (row-indexed copies, written by the paged pre-pass only).
// ... then the work-queue counters (8 per launch of at most kMaxSeqsPerLaunch
// sequences), from attn_workspace_ctr_offset, 256-byte aligned.
size_t attn_workspace_bytes(int Hkv, int R, bool fp8, int num_seqs);
size_t attn_workspace_ctr_offset(int Hkv, int R, bool fp8);
size_t attn_workspace_img16_offset(int Hkv, int R);
size_t attn_workspace_scales_offset(int Hkv, int R);
hipError_t launch_vprep(const AttnLaunch &a, bool fp8, hipStream_t s);
// Paged pre-pass for the rows of one launch's sequences.
hipError_t launch_vprep_paged(const AttnLaunch &a, const SeqTable &t, int rows_in_launch, int launch_index,
                              hipStream_t s);
// pv16 (fp8 only): every block's P.V with fp16 weights against the fp16 V^T image.
// launch_index: which launch of the call this is (its 8 work-queue counters).
hipError_t launch_attn(const AttnLaunch &a, const SeqTable &t, int rows_in_launch,
                       bool sparse, bool fp8, bool pv16, int launch_index, hipStream_t s);
// bf16 block-sparse attention over 64-query rows (lists [Hq][2R][k_cap]).
hipError_t launch_attn_q64(const AttnLaunch &a, const SeqTable &t, int rows_in_launch, int launch_index,
                           hipStream_t s);

}  // namespace stem
