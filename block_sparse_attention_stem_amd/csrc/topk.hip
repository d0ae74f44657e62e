// Stage 2 - Token-Position-Decay schedule and per-row top-k on gfx950.
//
// gist.science Stem summary §2.1: per query block I, budget k(I) =
// floor(ke - ke (1 - mu) I / nb), decaying linearly to mu * ke; AngelSlim doc
// §2.2: per-layer alpha, sink (initial) blocks and the sliding window always
// kept; zhichai summary §四 Step 2: top-k per query block.
//
// One wave per (head, query-block row).  Lane l holds candidates J = l + 64 m
// (m < 32, so rows up to 2048 blocks), i.e. ascending J runs over (m, lane).
// Scores become order-preserving unsigned keys (NaN -> the key of -inf, -0 ->
// the key of +0; forced and non-causal slots get key 0, below every real
// key).  The need-th largest key T is found MSB-first: a candidate threshold
// is counted with one vector compare per m whose result lands in a 64-bit
// scalar mask (ballot) and a scalar popcount, so no lane reduction is needed;
// the bits above the highest bit in which the row's smallest and largest keys
// differ are common to every key and are taken as given.  Then every key > T
// is taken and keys == T in ascending J until the budget is met: exactly
// "score descending, lower block index first".  The list is emitted ascending
// with ballot/mbcnt prefix counts (no sorting network).
#include "stem_internal.h"
#include "gfx950_util.h"

namespace stem {

constexpr int kPer = kMaxRowBlocks / 64;   // candidates per lane

__device__ __forceinline__ uint32_t order_key(float s) {
  if (s != s) s = -INFINITY;                       // NaN ranks as -inf
  s += 0.0f;                                       // -0 -> +0 (equal scores, equal keys)
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Wave-wide max / min of an unsigned value: within each row of 16 lanes by
// DPP (pairs, quads, half-row mirror, row mirror), then across the four rows
// through readlane; the result is uniform.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_get(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t umax2(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin2(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = umax2(x, dpp_get<0xB1>(x));
  x = umax2(x, dpp_get<0x4E>(x));
  x = umax2(x, dpp_get<0x141>(x));
  x = umax2(x, dpp_get<0x140>(x));
  return umax2(umax2((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
               umax2((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
  x = umin2(x, dpp_get<0xB1>(x));
  x = umin2(x, dpp_get<0x4E>(x));
  x = umin2(x, dpp_get<0x141>(x));
  x = umin2(x, dpp_get<0x140>(x));
  return umin2(umin2((uint32_t)__builtin_amdgcn_readlane((int)x, 0), (uint32_t)__builtin_amdgcn_readlane((int)x, 16)),
               umin2((uint32_t)__builtin_amdgcn_readlane((int)x, 32), (uint32_t)__builtin_amdgcn_readlane((int)x, 48)));
}

// One row with candidates in MC slots per lane (J = lane + 64 m, m < MC;
// slots past the row hold key 0).  MC is a compile-time bound, so no loop
// over the slots carries a per-slot guard: a guard is a scalar compare and
// branch, and with one scalar unit per CU they were most of the kernel's
// time.
template <int MC>
__device__ __forceinline__ void topk_row(const float *__restrict__ srow, int32_t *__restrict__ orow,
                                         int32_t *__restrict__ ocnt, int k_cap, int I, int sink_end, int win0,
                                         int need, int n_cand, int lane) {
  // Every slot's score is requested before any is used (slots past the row
  // re-read entry I, which exists): loads placed inside the per-slot
  // conditions below were each awaited before the next one was issued.
  float sv[MC];
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const int J = lane + 64 * m;
    sv[m] = srow[J <= I ? J : I];
  }
  uint32_t key[MC];
  uint32_t forced = 0;                             // bit m: forced block
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    key[m] = 0;
    const int J = lane + 64 * m;
    if (J <= I) {
      if ((J < sink_end) || (J >= win0)) forced |= 1u << m;
      else {
        key[m] = order_key(sv[m]);
        kmax = key[m] > kmax ? key[m] : kmax;
        kmin = key[m] < kmin ? key[m] : kmin;
      }
    }
  }

  uint32_t sel = 0;                                // bit m: selected candidate
  if (need >= n_cand) {
#pragma unroll
    for (int m = 0; m < MC; ++m)
      if (key[m] != 0u) sel |= 1u << m;
  } else if (need > 0) {
    // Every candidate key lies in [lo, hi], so all of them (and T) share the
    // bits of lo above the highest bit in which lo and hi differ.
    const uint32_t hi = wave_umax(kmax), lo = wave_umin(kmin);
    uint32_t T = lo;
    if (hi != lo) {
      const int top = 31 - __builtin_clz(hi ^ lo);
      T = top == 31 ? 0u : (lo & ~((2u << top) - 1u));
      // Invariant: c_T = count(key >= T) >= need.  Once c_T == need the
      // selected set is fixed (every key >= T), so the lower bits of T are
      // not needed; on continuous scores that happens after about
      // log2(n_cand) bits, not all of them.
      int c_T = n_cand;
      for (int bit = top; bit >= 0 && c_T != need; --bit) {
        const uint32_t cand = T | (1u << bit);
        int c = 0;
#pragma unroll
        for (int m = 0; m < MC; ++m) c += __popcll(__ballot(key[m] >= cand));
        if (c >= need) {
          T = cand;
          c_T = c;
        }
      }
    }
    // T >= 1 and count(key >= T) >= need, with equality unless T is exactly
    // the need-th largest key (ties): key 0 (no candidate) never counts
    int c_gt = 0;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      const uint64_t gm = __ballot(key[m] > T);
      if ((gm >> lane) & 1u) sel |= 1u << m;
      c_gt += __popcll(gm);
    }
    const int take_eq = need - c_gt;
    int taken = 0;
#pragma unroll
    for (int m = 0; m < MC; ++m) {
      if (taken < take_eq) {
        const uint64_t em = __ballot(key[m] == T);
        if (((em >> lane) & 1u) && taken + lanes_below(em) < take_eq) sel |= 1u << m;
        taken += __popcll(em);
      }
    }
  }

  int base = 0;
#pragma unroll
  for (int m = 0; m < MC; ++m) {
    const bool in = ((forced | sel) >> m) & 1u;
    const uint64_t im = __ballot(in);
    const int pos = base + lanes_below(im);
    if (in && pos < k_cap) orow[pos] = lane + 64 * m;
    base += __popcll(im);
  }
  for (int p = base + lane; p < k_cap; p += 64) orow[p] = -1;
  if (lane == 0) *ocnt = base;
}

// kMaxMC: the most slots any row of the launch needs (16 for rows of at
// most 1024 blocks, else 32); the narrower instance needs fewer registers,
// so more waves share each SIMD.
template <int kMaxMC>
__global__ __launch_bounds__(256) void topk_kernel(TopkLaunch a, SeqTable t, int rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = blockIdx.x * 4 + wave;
  if (item >= rows * a.Hq) return;
  const int h = item % a.Hq;
  // rows in descending order: the longest rows (most slots) start first, so
  // the short ones fill the tail of the launch
  const int rl = rows - 1 - item / a.Hq;           // row within this launch
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

  const float *srow = a.scores + ((size_t)h * a.R + r) * a.max_nb;
  int32_t *orow = a.idx + ((size_t)h * a.R + r) * a.k_cap;
  int32_t *ocnt = a.cnt + (size_t)h * a.R + r;
  // slots per lane: J <= I needs m <= I / 64; rounded up to a multiple of 4
  switch ((I >> 8) + 1) {
    case 1: topk_row<4>(srow, orow, ocnt, a.k_cap, I, sink_end, win0, need, n_cand, lane); break;
    case 2: topk_row<8>(srow, orow, ocnt, a.k_cap, I, sink_end, win0, need, n_cand, lane); break;
    case 3: topk_row<12>(srow, orow, ocnt, a.k_cap, I, sink_end, win0, need, n_cand, lane); break;
    case 4: topk_row<16>(srow, orow, ocnt, a.k_cap, I, sink_end, win0, need, n_cand, lane); break;
    default:
      if constexpr (kMaxMC > 16) {
        switch ((I >> 8) + 1) {
          case 5: topk_row<20>(srow, orow, ocnt, a.k_cap, I, sink_end, win0, need, n_cand, lane); break;
          case 6: topk_row<24>(srow, orow, ocnt, a.k_cap, I, sink_end, win0, need, n_cand, lane); break;
          case 7: topk_row<28>(srow, orow, ocnt, a.k_cap, I, sink_end, win0, need, n_cand, lane); break;
          default: topk_row<kPer>(srow, orow, ocnt, a.k_cap, I, sink_end, win0, need, n_cand, lane); break;
        }
      }
      break;
  }
}

hipError_t launch_topk(const TopkLaunch &a, const SeqTable &t, int rows, hipStream_t s) {
  const int waves = rows * a.Hq;
  int max_nb = 0;
  for (int z = 0; z < t.n; ++z) max_nb = t.row[z + 1] - t.row[z] > max_nb ? t.row[z + 1] - t.row[z] : max_nb;
  if (max_nb <= 1024) hipLaunchKernelGGL(topk_kernel<16>, dim3((waves + 3) / 4), dim3(256), 0, s, a, t, rows);
  else hipLaunchKernelGGL(topk_kernel<kPer>, dim3((waves + 3) / 4), dim3(256), 0, s, a, t, rows);
  return hipGetLastError();
}

}  // namespace stem
