// C ABI of the Stem sparse-prefill library (declared in include/stem.h).
// Validation happens on the host before anything is enqueued; kernels get
// the packed-batch offsets by value, up to 64 sequences per launch.
#include "stem.h"
#include "stem_internal.h"

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

using namespace stem;

namespace {

struct Shape {
  int B, Hq, Hkv, T, R, max_nb;
};

int check_problem(const stem_problem_t *p, Shape *s) {
  if (!p || !p->cu_seqlens_host || p->num_seqs < 1) return STEM_ERR_INVALID_ARG;
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1 || p->block_size < 1)
    return STEM_ERR_INVALID_ARG;
  if (p->num_q_heads % p->num_kv_heads != 0) return STEM_ERR_INVALID_ARG;
  if (p->head_dim != kHeadDim || p->block_size != kBlock) return STEM_ERR_UNSUPPORTED;
  const int32_t *cu = p->cu_seqlens_host;
  if (cu[0] != 0) return STEM_ERR_INVALID_ARG;
  int max_nb = 0;
  for (int z = 0; z < p->num_seqs; ++z) {
    const int64_t L = (int64_t)cu[z + 1] - cu[z];
    if (L <= 0) return STEM_ERR_INVALID_ARG;
    if (L % kBlock != 0) return STEM_ERR_UNSUPPORTED;   // ragged tail block
    if (L / kBlock > max_nb) max_nb = (int)(L / kBlock);
  }
  const int64_t T = cu[p->num_seqs];
  s->B = p->num_seqs;
  s->Hq = p->num_q_heads;
  s->Hkv = p->num_kv_heads;
  s->T = (int)T;
  s->R = (int)(T / kBlock);
  s->max_nb = max_nb;
  return STEM_OK;
}

// Fill the table for sequences [z0, z0 + n).
void fill_table(const stem_problem_t *p, int z0, int n, SeqTable *t) {
  memset(t, 0, sizeof(*t));
  t->n = n;
  t->z0 = z0;
  for (int i = 0; i <= n; ++i) {
    t->tok[i] = p->cu_seqlens_host[z0 + i];
    t->row[i] = t->tok[i] / kBlock;
  }
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char *stem_status_string(int status) {
  switch (status) {
    case STEM_OK: return "STEM_OK";
    case STEM_ERR_INVALID_ARG: return "STEM_ERR_INVALID_ARG";
    case STEM_ERR_UNSUPPORTED: return "STEM_ERR_UNSUPPORTED";
    case STEM_ERR_CAPACITY: return "STEM_ERR_CAPACITY";
    case STEM_ERR_WORKSPACE: return "STEM_ERR_WORKSPACE";
    case STEM_ERR_HIP: return "STEM_ERR_HIP";
    default: return "STEM_ERR_UNKNOWN";
  }
}

size_t stem_score_workspace_bytes(const stem_problem_t *p) {
  Shape s;
  if (check_problem(p, &s) != STEM_OK) return 0;
  // per (KV head, key block): log value norm, then the bonus (fp32); then
  // the scoring kernel's work-queue counters
  return score_workspace_bytes(s.Hkv, s.R, s.B);
}

}  // extern "C"

static int score_common(const stem_problem_t *p, const void *q, const void *k, const void *v,
                        const float *q_scale, const float *k_scale, const float *v_scale, bool fp8,
                        int32_t stride, int32_t chunk_size, float norm, float beta, float *scores,
                        void *workspace, size_t workspace_bytes, void *stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st != STEM_OK) return st;
  if (!q || !k || !v || !scores) return STEM_ERR_INVALID_ARG;
  if (fp8 && (!q_scale || !k_scale || !v_scale)) return STEM_ERR_INVALID_ARG;
  if (stride < 1 || kBlock % stride != 0) return STEM_ERR_INVALID_ARG;
  if (stride != 8) return STEM_ERR_UNSUPPORTED;
  if (chunk_size < kBlock || chunk_size % kBlock != 0) return STEM_ERR_INVALID_ARG;
  if (!(norm > 0.f) || !isfinite(norm) || !isfinite(beta) || beta < 0.f) return STEM_ERR_INVALID_ARG;
  if (s.max_nb > kMaxScoreBlocks) return STEM_ERR_UNSUPPORTED;
  const size_t need = stem_score_workspace_bytes(p);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return STEM_ERR_WORKSPACE;

  ScoreLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.fp8 = fp8;
  a.scores = scores;
  a.ell = (float *)workspace;
  a.ctr = (int32_t *)((uint8_t *)workspace + score_workspace_ctr_offset(s.Hkv, s.R));
  a.n_ctr = 8 * ((s.B + kMaxSeqsPerLaunch - 1) / kMaxSeqsPerLaunch);
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.R = s.R;
  a.max_nb = s.max_nb;
  a.stride = stride;
  a.chunk_size = chunk_size;
  a.scale = (float)(1.0 / (sqrt((double)kHeadDim) * stride * (double)norm));
  a.beta = beta;
  hipStream_t hs = as_stream(stream);

  if (launch_vnorm(a, hs) != hipSuccess) return STEM_ERR_HIP;
  for (int z0 = 0; z0 < s.B; z0 += kMaxSeqsPerLaunch) {
    const int n = s.B - z0 < kMaxSeqsPerLaunch ? s.B - z0 : kMaxSeqsPerLaunch;
    SeqTable t;
    fill_table(p, z0, n, &t);
    if (launch_vstats(a, t, hs) != hipSuccess) return STEM_ERR_HIP;
  }
  // Score tiles: per sequence, Hkv x (tiles of the causal triangle) slots,
  // each run for the G query heads of the group.  chunk_size only names the
  // query-axis tiling of the pages; it changes no value and the kernel's
  // own tiles replace it.
  const int G = s.Hq / s.Hkv;
  for (int z0 = 0; z0 < s.B; z0 += kMaxSeqsPerLaunch) {
    const int n = s.B - z0 < kMaxSeqsPerLaunch ? s.B - z0 : kMaxSeqsPerLaunch;
    SeqTable t;
    fill_table(p, z0, n, &t);
    int64_t slots = 0;
    for (int i = 0; i < n; ++i) {
      t.item[i] = (int32_t)slots;
      const int nb = t.row[i + 1] - t.row[i];
      slots += (int64_t)s.Hkv * score_pairs(nb);
    }
    t.item[n] = (int32_t)slots;
    const int64_t items = slots * G;
    if (items >= ((int64_t)1 << 31)) return STEM_ERR_UNSUPPORTED;
    if (launch_score(a, t, (int)items, z0 / kMaxSeqsPerLaunch, hs) != hipSuccess) return STEM_ERR_HIP;
  }
  return STEM_OK;
}


// ------------------------------------------------------------ no-alloc path
// stem_score_noalloc uses this file-scope device array in place of the
// caller's score workspace.  Each GPU the library runs on holds its own copy
// (at its own address) until the process ends.  In host code the name
// `scratch` is only a stand-in for the symbol: its device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// only that address is ever passed to a kernel.
static __device__ __attribute__((aligned(256))) uint8_t scratch[STEM_SCORE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];    // device address of `scratch` per device, null until resolved

// The device `stream` launches on (the current device for the null stream),
// and that device's address of `scratch`, resolved on first use.
int scratch_for_stream(hipStream_t stream, void **out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return STEM_ERR_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return STEM_ERR_HIP;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return STEM_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return STEM_ERR_HIP;
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !ptr || ((uintptr_t)ptr & 255u)) return STEM_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return STEM_OK;
}
}  // namespace

extern "C" {

int stem_score(const stem_problem_t *p, const void *q, const void *k, const void *v,
               int32_t stride, int32_t chunk_size, float norm, float beta, float *scores,
               void *workspace, size_t workspace_bytes, void *stream) {
  return score_common(p, q, k, v, nullptr, nullptr, nullptr, false, stride, chunk_size, norm, beta, scores,
                      workspace, workspace_bytes, stream);
}

int stem_score_noalloc(const stem_problem_t *p, const void *q, const void *k, const void *v,
                       int32_t stride, int32_t chunk_size, float norm, float beta, float *scores,
                       void *stream) {
  // the size check comes first, so an oversized problem never touches the device
  Shape s;
  const int st = check_problem(p, &s);
  if (st != STEM_OK) return st;
  if (stem_score_workspace_bytes(p) > (size_t)STEM_SCORE_SCRATCH_BYTES) return STEM_ERR_WORKSPACE;
  void *ptr = nullptr;
  const int sr = scratch_for_stream(as_stream(stream), &ptr);
  if (sr != STEM_OK) return sr;
  return score_common(p, q, k, v, nullptr, nullptr, nullptr, false, stride, chunk_size, norm, beta, scores, ptr,
                      (size_t)STEM_SCORE_SCRATCH_BYTES, stream);
}

int stem_score_fp8(const stem_problem_t *p, const void *q, const void *k, const void *v,
                   const float *q_scale, const float *k_scale, const float *v_scale, int32_t stride,
                   int32_t chunk_size, float norm, float beta, float *scores, void *workspace,
                   size_t workspace_bytes, void *stream) {
  return score_common(p, q, k, v, q_scale, k_scale, v_scale, true, stride, chunk_size, norm, beta, scores,
                      workspace, workspace_bytes, stream);
}

int32_t stem_tpd_budget(int32_t I, int32_t nb, double k_start, double mu, double alpha) {
  if (nb <= 0 || I < 0) return 0;
  return tpd_budget(I, nb, alpha * k_start, mu);
}

int32_t stem_kept_count(int32_t I, int32_t nb, double k_start, double mu, double alpha,
                        int32_t n_init, int32_t n_window) {
  if (nb <= 0 || I < 0) return 0;
  return kept_count(I, nb, alpha * k_start, mu, n_init, n_window);
}

int32_t stem_max_kept(const stem_problem_t *p, const double *k_start_host, double mu,
                      double alpha, int32_t n_init, int32_t n_window) {
  Shape s;
  if (check_problem(p, &s) != STEM_OK || !k_start_host) return -1;
  int best = 0;
  for (int z = 0; z < s.B; ++z) {
    const int nb = (p->cu_seqlens_host[z + 1] - p->cu_seqlens_host[z]) / kBlock;
    const double ke = alpha * k_start_host[z];
    for (int I = 0; I < nb; ++I) {
      const int kc = kept_count(I, nb, ke, mu, n_init, n_window);
      if (kc > best) best = kc;
    }
  }
  return best;
}

int stem_schedule_topk(const stem_problem_t *p, const float *scores, const double *k_start_host,
                       double mu, double alpha, int32_t n_init, int32_t n_window, int32_t k_cap,
                       int32_t *block_idx, int32_t *block_cnt, void *stream) {
  Shape s;
  int st = check_problem(p, &s);
  if (st != STEM_OK) return st;
  if (!scores || !k_start_host || !block_idx || !block_cnt) return STEM_ERR_INVALID_ARG;
  if (!(mu > 0.0 && mu <= 1.0) || !(alpha > 0.0) || !isfinite(alpha)) return STEM_ERR_INVALID_ARG;
  if (n_init < 0 || n_window < 0 || k_cap < 1) return STEM_ERR_INVALID_ARG;
  for (int z = 0; z < s.B; ++z)
    if (!(k_start_host[z] >= 0.0) || !isfinite(k_start_host[z])) return STEM_ERR_INVALID_ARG;
  if (s.max_nb > kMaxRowBlocks) return STEM_ERR_UNSUPPORTED;
  const int need = stem_max_kept(p, k_start_host, mu, alpha, n_init, n_window);
  if (k_cap < need) return STEM_ERR_CAPACITY;

  TopkLaunch a;
  memset(&a, 0, sizeof(a));
  a.scores = scores;
  a.idx = block_idx;
  a.cnt = block_cnt;
  a.Hq = s.Hq;
  a.R = s.R;
  a.max_nb = s.max_nb;
  a.k_cap = k_cap;
  a.mu = mu;
  a.n_init = n_init;
  a.n_window = n_window;
  hipStream_t hs = as_stream(stream);
  for (int z0 = 0; z0 < s.B; z0 += kMaxSeqsPerLaunch) {
    const int n = s.B - z0 < kMaxSeqsPerLaunch ? s.B - z0 : kMaxSeqsPerLaunch;
    SeqTable t;
    fill_table(p, z0, n, &t);
    for (int i = 0; i < n; ++i) a.ke[i] = alpha * k_start_host[z0 + i];
    if (launch_topk(a, t, t.row[n] - t.row[0], hs) != hipSuccess) return STEM_ERR_HIP;
  }
  return STEM_OK;
}

size_t stem_attn_workspace_bytes(const stem_problem_t *p, int32_t dtype) {
  Shape s;
  if (check_problem(p, &s) != STEM_OK) return 0;
  if (dtype != STEM_DTYPE_BF16 && dtype != STEM_DTYPE_FP8_E4M3 && dtype != STEM_DTYPE_FP8_E4M3_PV16) return 0;
  return attn_workspace_bytes(s.Hkv, s.R, dtype != STEM_DTYPE_BF16, s.B);
}

static int attn_common(const stem_problem_t *p, int32_t dtype, const void *q, const void *k,
                       const void *v, const float *q_scale, const float *k_scale,
                       const float *v_scale, const int32_t *block_idx, const int32_t *block_cnt,
                       int32_t k_cap, float softmax_scale, void *out, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream, bool sparse,
                       const int32_t *table = nullptr, int32_t table_stride = 0, int32_t num_pages = 0,
                       bool q64 = false) {
  Shape s;
  int st = check_problem(p, &s);
  if (st != STEM_OK) return st;
  if (!q || !k || !v || !out) return STEM_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return STEM_ERR_INVALID_ARG;
  bool fp8, pv16 = false;
  if (dtype == STEM_DTYPE_BF16) {
    if (q_scale || k_scale || v_scale) return STEM_ERR_INVALID_ARG;
    fp8 = false;
  } else if (dtype == STEM_DTYPE_FP8_E4M3 || dtype == STEM_DTYPE_FP8_E4M3_PV16) {
    if (!q_scale || !k_scale || !v_scale) return STEM_ERR_INVALID_ARG;
    fp8 = true;
    pv16 = dtype == STEM_DTYPE_FP8_E4M3_PV16;
  } else {
    return STEM_ERR_UNSUPPORTED;
  }
  if (sparse && (!block_idx || !block_cnt || k_cap < 1)) return STEM_ERR_INVALID_ARG;
  if (q64 && s.max_nb > kMaxListBlocks) return STEM_ERR_UNSUPPORTED;
  const size_t need = attn_workspace_bytes(s.Hkv, s.R, fp8, s.B);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)) return STEM_ERR_WORKSPACE;

  AttnLaunch a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.idx = block_idx;
  a.cnt = block_cnt;
  a.k_cap = k_cap;
  a.out = out;
  a.lse = lse;
  if (fp8) {
    // the fp16 V^T image is read only with fp16 weights; the pre-pass skips it otherwise
    a.vimg8 = (uint8_t *)workspace;
    a.vimg16 = pv16 ? (uint16_t *)((uint8_t *)workspace + attn_workspace_img16_offset(s.Hkv, s.R)) : nullptr;
  } else {
    a.vimg8 = nullptr;
    a.vimg16 = (uint16_t *)workspace;
  }
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.R = s.R;
  a.T = s.T;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  a.table = table;
  a.table_stride = table_stride;
  a.num_pages = num_pages;
  a.k_scale_pages = nullptr;
  a.v_scale_pages = nullptr;
  if (table) {
    // the paged pre-pass copies page scales to row-indexed arrays
    float *rs = (float *)((uint8_t *)workspace + attn_workspace_scales_offset(s.Hkv, s.R));
    a.k_scale_pages = k_scale;
    a.v_scale_pages = v_scale;
    a.k_scale = rs;
    a.v_scale = rs + (size_t)s.R * s.Hkv;
  }
  a.ctr = (int32_t *)((uint8_t *)workspace + attn_workspace_ctr_offset(s.Hkv, s.R, fp8));
  a.n_ctr = 8 * ((s.B + kMaxSeqsPerLaunch - 1) / kMaxSeqsPerLaunch);
  hipStream_t hs = as_stream(stream);
  if (!table && launch_vprep(a, fp8, hs) != hipSuccess) return STEM_ERR_HIP;
  for (int z0 = 0; z0 < s.B; z0 += kMaxSeqsPerLaunch) {
    const int n = s.B - z0 < kMaxSeqsPerLaunch ? s.B - z0 : kMaxSeqsPerLaunch;
    SeqTable t;
    fill_table(p, z0, n, &t);
    const int rows = t.row[n] - t.row[0];
    if ((int64_t)rows * s.Hq >= ((int64_t)1 << 31)) return STEM_ERR_UNSUPPORTED;
    const int li = z0 / kMaxSeqsPerLaunch;
    if (table && launch_vprep_paged(a, t, rows, li, hs) != hipSuccess) return STEM_ERR_HIP;
    const hipError_t e =
        q64 ? launch_attn_q64(a, t, rows, li, hs) : launch_attn(a, t, rows, sparse, fp8, pv16, li, hs);
    if (e != hipSuccess) return STEM_ERR_HIP;
  }
  return STEM_OK;
}

int stem_bsa_prefill(const stem_problem_t *p, int32_t dtype, const void *q, const void *k,
                     const void *v, const float *q_scale, const float *k_scale,
                     const float *v_scale, const int32_t *block_idx, const int32_t *block_cnt,
                     int32_t k_cap, float softmax_scale, void *out, float *lse, void *workspace,
                     size_t workspace_bytes, void *stream) {
  return attn_common(p, dtype, q, k, v, q_scale, k_scale, v_scale, block_idx, block_cnt, k_cap,
                     softmax_scale, out, lse, workspace, workspace_bytes, stream, true);
}

int stem_dense_prefill(const stem_problem_t *p, int32_t dtype, const void *q, const void *k,
                       const void *v, const float *q_scale, const float *k_scale,
                       const float *v_scale, float softmax_scale, void *out, float *lse,
                       void *workspace, size_t workspace_bytes, void *stream) {
  return attn_common(p, dtype, q, k, v, q_scale, k_scale, v_scale, nullptr, nullptr, 0,
                     softmax_scale, out, lse, workspace, workspace_bytes, stream, false);
}

int stem_bsa_prefill_q64(const stem_problem_t *p, const void *q, const void *k, const void *v,
                         const int32_t *block_idx, const int32_t *block_cnt, int32_t k_cap,
                         float softmax_scale, void *out, float *lse, void *workspace,
                         size_t workspace_bytes, void *stream) {
  return attn_common(p, STEM_DTYPE_BF16, q, k, v, nullptr, nullptr, nullptr, block_idx, block_cnt, k_cap,
                     softmax_scale, out, lse, workspace, workspace_bytes, stream, true, nullptr, 0, 0, true);
}

int stem_bsa_prefill_paged(const stem_problem_t *p, const void *q, const void *k_pages,
                           const void *v_pages, const float *q_scale, const float *k_scale_pages,
                           const float *v_scale_pages, const int32_t *block_table,
                           int32_t table_stride, int32_t num_pages, const int32_t *block_idx,
                           const int32_t *block_cnt, int32_t k_cap, float softmax_scale, void *out,
                           float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  Shape s;
  const int st = check_problem(p, &s);
  if (st != STEM_OK) return st;
  if (!block_table || num_pages < 1 || table_stride < s.max_nb) return STEM_ERR_INVALID_ARG;
  return attn_common(p, STEM_DTYPE_FP8_E4M3, q, k_pages, v_pages, q_scale, k_scale_pages, v_scale_pages,
                     block_idx, block_cnt, k_cap, softmax_scale, out, lse, workspace, workspace_bytes, stream,
                     true, block_table, table_stride, num_pages);
}

}  // extern "C"
