// Stage 2 - Token-Position-Decay schedule and per-row top-k on gfx950.
//
// gist.science Stem summary §2.1: per query block I, budget k(I) =
// floor(ke - ke (1 - mu) I / nb), decaying linearly to mu * ke; AngelSlim doc
// §2.2: per-layer alpha, sink (initial) blocks and the sliding window always
// kept; zhichai summary §四 Step 2: top-k per query block.
//
// One wave per (head, query-block row).  Lane l holds candidates J = l + 64 m
// (m < 32, so rows up to 2048 blocks), i.e. ascending J runs over (m, lane).
// Scores become order-preserving unsigned keys (NaN -> the key of -inf); the
// need-th largest key T is found MSB-first with wave-wide counts, then every
// key > T is taken and keys == T are taken in ascending J until the budget is
// met: exactly "score descending, lower block index first".  The list is
// emitted ascending with ballot/mbcnt prefix counts (no sorting network).
#include "stem_internal.h"
#include "gfx950_util.h"

namespace stem {

constexpr int kPer = kMaxRowBlocks / 64;   // candidates per lane

__device__ __forceinline__ uint32_t order_key(float s) {
  if (s != s) s = -INFINITY;                       // NaN ranks as -inf
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__global__ __launch_bounds__(256) void topk_kernel(TopkLaunch a, SeqTable t, int rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = blockIdx.x * 4 + wave;
  if (item >= rows * a.Hq) return;
  const int h = item % a.Hq;
  const int rl = item / a.Hq;                      // row within this launch
  const int r = t.row[0] + rl;                     // global row
  const int z = seq_of(t.row, t.n, r);
  const int I = r - t.row[z];
  const int nb = t.row[z + 1] - t.row[z];

  const int kept = kept_count(I, nb, a.ke[z], a.mu, a.n_init, a.n_window);
  const int sink_end = a.n_init < I + 1 ? a.n_init : I + 1;
  int win0 = I - a.n_window + 1;
  if (a.n_window <= 0) win0 = I + 1;
  if (win0 < 0) win0 = 0;
  const int n_forced = forced_count(I, a.n_init, a.n_window);
  const int need = kept - n_forced;
  const int n_cand = I + 1 - n_forced;
  const int mcount = (I + 64) >> 6;                // lanes hold J < 64 * mcount

  const float *srow = a.scores + ((size_t)h * a.R + r) * a.max_nb;
  uint32_t key[kPer];
  uint32_t valid = 0, forced = 0;                  // bit m: candidate / forced
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    key[m] = 0;
    if (m < mcount) {
      const int J = lane + 64 * m;
      if (J <= I) {
        const bool f = (J < sink_end) || (J >= win0);
        if (f) forced |= 1u << m;
        else {
          valid |= 1u << m;
          key[m] = order_key(srow[J]);
        }
      }
    }
  }

  uint32_t sel = 0;
  if (need >= n_cand) {
    sel = valid;
  } else if (need > 0) {
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int c = 0;
#pragma unroll
      for (int m = 0; m < kPer; ++m)
        if (m < mcount) c += ((valid >> m) & 1u) && key[m] >= cand;
      if (wave_sum(c) >= need) T = cand;
    }
    int c_gt = 0;
#pragma unroll
    for (int m = 0; m < kPer; ++m)
      if (m < mcount && ((valid >> m) & 1u) && key[m] > T) {
        sel |= 1u << m;
        ++c_gt;
      }
    const int take_eq = need - wave_sum(c_gt);
    int taken = 0;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      if (m < mcount) {
        const bool eq = ((valid >> m) & 1u) && key[m] == T;
        const uint64_t em = __ballot(eq);
        if (eq && taken + lanes_below(em) < take_eq) sel |= 1u << m;
        taken += __popcll(em);
      }
    }
  }

  int32_t *orow = a.idx + ((size_t)h * a.R + r) * a.k_cap;
  int base = 0;
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    if (m < mcount) {
      const bool in = ((forced | sel) >> m) & 1u;
      const uint64_t im = __ballot(in);
      const int pos = base + lanes_below(im);
      if (in && pos < a.k_cap) orow[pos] = lane + 64 * m;
      base += __popcll(im);
    }
  }
  for (int p = base + lane; p < a.k_cap; p += 64) orow[p] = -1;
  if (lane == 0) a.cnt[(size_t)h * a.R + r] = base;
}

hipError_t launch_topk(const TopkLaunch &a, const SeqTable &t, int rows, hipStream_t s) {
  const int waves = rows * a.Hq;
  hipLaunchKernelGGL(topk_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, a, t, rows);
  return hipGetLastError();
}

}  // namespace stem
