// Stage 1 - block scoring on gfx950.
//
// AngelSlim doc "Stem: Rethinking Causal Information Flow in Sparse
// Attention" §2.1: score(Q_i, K_j) = Q_i.K_j^T / (sqrt(d) s n) + lambda
// ReLU(vbar_j), from a strided group GEMM (stride s); gist.science Stem
// summary §2.2-2.3: anti-diagonal down-sampling of Q.K^T, block-wise max
// pooling, value magnitude from block max pooling.
//
// Three kernels:
//   vnorm   l[g][kb] = ln max_{t in key block kb} ||V[t][g]||^2     (HBM scan)
//   vstats  bonus = beta * max(0, zscore(l)) per (sequence, KV head)
//   score   strided anti-diagonal GEMM on bf16 MFMA, with the causal mask,
//           the 16x16 max-pool, the 1/(sqrt(d) s n) scale and the bonus fused
//           into the epilogue.  Only the causal triangle of 256x128 strided
//           tiles is launched; scores never touch HBM before pooling.
#include <utility>

#include "stem_internal.h"
#include "gfx950_util.h"

namespace stem {

// ------------------------------------------------------------------ vnorm
// One workgroup per (global key block, KV head); 16 lanes per token row
// (16 x 16 B = 256 B = one head vector), 16 rows per pass.
__global__ __launch_bounds__(256) void vnorm_kernel(const __bf16 *__restrict__ v,
                                                    float *__restrict__ ell, int Hkv, int R) {
  const int kb = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, sub = tid & 15, rowg = tid >> 4;
  __shared__ float red[16];
  float emax = 0.f;
  for (int t = rowg; t < kBlock; t += 16) {
    const size_t tok = (size_t)kb * kBlock + t;
    const u32x4 raw = ld16(v + (tok * Hkv + g) * kHeadDim + sub * 8);
    float e = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = __uint_as_float(raw[w] << 16);
      const float hi = __uint_as_float(raw[w] & 0xffff0000u);
      e = fmaf(lo, lo, e);
      e = fmaf(hi, hi, e);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) e += __shfl_xor(e, o, 64);
    emax = fmaxf(emax, e);
  }
  if (sub == 0) red[rowg] = emax;
  __syncthreads();
  if (tid == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) m = fmaxf(m, red[i]);
    ell[(size_t)g * R + kb] = logf(fmaxf(m, 1e-30f));
  }
}

hipError_t launch_vnorm(const ScoreLaunch &a, hipStream_t s) {
  dim3 grid(a.R, a.Hkv);
  hipLaunchKernelGGL(vnorm_kernel, grid, dim3(256), 0, s, (const __bf16 *)a.v, a.ell, a.Hkv, a.R);
  return hipGetLastError();
}

// ------------------------------------------------------------------ vstats
// One workgroup per (sequence, KV head): mean and population std of l over
// the sequence's key blocks (fp64 sums), then bonus written in place.
__global__ __launch_bounds__(256) void vstats_kernel(float *__restrict__ ell, SeqTable t,
                                                     int R, float beta) {
  const int z = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int r0 = t.row[z], nb = t.row[z + 1] - t.row[z];
  float *e = ell + (size_t)g * R + r0;
  __shared__ double red[2][256];
  double s1 = 0.0, s2 = 0.0;
  for (int j = tid; j < nb; j += 256) s1 += (double)e[j];
  red[0][tid] = s1;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[0][tid] += red[0][tid + o];
    __syncthreads();
  }
  const double mean = red[0][0] / nb;
  for (int j = tid; j < nb; j += 256) {
    const double dv = (double)e[j] - mean;
    s2 += dv * dv;
  }
  red[1][tid] = s2;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[1][tid] += red[1][tid + o];
    __syncthreads();
  }
  const double sd = sqrt(red[1][0] / nb);
  const double inv = 1.0 / (sd + 1e-6);
  for (int j = tid; j < nb; j += 256) {
    const double zs = ((double)e[j] - mean) * inv;
    e[j] = (float)((double)beta * (zs > 0.0 ? zs : 0.0));
  }
}

hipError_t launch_vstats(const ScoreLaunch &a, const SeqTable &t, hipStream_t s) {
  dim3 grid(t.n, a.Hkv);
  hipLaunchKernelGGL(vstats_kernel, grid, dim3(256), 0, s, a.ell, t, a.R, a.beta);
  return hipGetLastError();
}

// ------------------------------------------------------------------ score
// Workgroup tile: 256 strided query rows x 128 strided key rows (= 16 x 8
// blocks of 16 strided rows), K = s*d = 1024 walked in 16 chunks of 64.
// Row i of the A matrix is Q[tok + i*s + t][h][:] for t = 0..s-1; row j of B
// is K[tok + j*s + (s-1-t)][g][:] (the anti-diagonal pairing).  Chunk c
// covers t = c / 2 and head dims (c % 2) * 64 .. +63: one 128-byte piece of
// one token row per matrix row.
//
// Eight waves (two per SIMD) in a 4 x 2 grid, each 64 x 64 = 2 x 2 MFMA 32x32
// tiles.  Chunks arrive by direct-to-LDS buffer loads into a ring of three
// stages (separate LDS arrays, the chunk loop fully unrolled), requested two
// chunks ahead: one barrier per chunk, no staging registers.  LDS rows are
// 128 bytes; a row's 16-byte pieces are stored XOR-permuted by (row / 2) % 8,
// so the 32 x 16-byte fragment reads of an MFMA hit every bank once.  The
// permutation is applied on the global side of the loads (each lane fetches
// the piece that belongs at its fixed LDS slot).
constexpr int kRowsA = 256;                 // strided query rows per tile
constexpr int kRowsB = 128;                 // strided key rows per tile
constexpr int kScoreBK = 64;                // K elements per chunk
constexpr int kChunks = 8 * kHeadDim / kScoreBK;   // 16
constexpr uint32_t kScoreBufWord3 = 0x00020000u;   // raw buffer descriptor word 3 (gfx9 dword access)

struct ScoreArgs {
  const __bf16 *q, *k;
  const float *bonus;
  float *scores;
  int32_t Hq, Hkv, R, max_nb, G;
  float scale;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Tile pair p of a (sequence, head) -> (row band ti, column band tj); band
// ti starts at pair ti (ti + 1) (see score_pairs).
__device__ __forceinline__ void band_decode(int p, int &ti, int &tj) {
  int r = (int)((sqrtf(4.f * (float)p + 1.f) - 1.f) * 0.5f);
  while ((r + 1) * (r + 2) <= p) ++r;
  while (r * (r + 1) > p) --r;
  ti = r;
  tj = p - r * (r + 1);
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt[3:0] | expcnt 7 | lgkmcnt 15 | vmcnt[5:4]).
template <int N>
__device__ __forceinline__ void score_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Barrier that waits for this wave's LDS reads but not for its loads in flight.
__device__ __forceinline__ void score_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename F, int... Is>
__device__ __forceinline__ void score_static_for_impl(F &&f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void score_static_for(F &&f) {
  score_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__global__ __launch_bounds__(512, 1) void score_kernel(ScoreArgs a, SeqTable t, int n_items) {
  __shared__ __attribute__((aligned(1024))) uint16_t A0[kRowsA * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t A1[kRowsA * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t A2[kRowsA * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t B0[kRowsB * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t B1[kRowsB * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t B2[kRowsB * kScoreBK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int item = xcd_chunk_item(blockIdx.x, n_items);
  const int slot = item / a.G, hh = item - slot * a.G;
  // slot -> (sequence, KV head, tile); item prefix counts slots
  const int z = seq_of(t.item, t.n, slot);
  const int local = slot - t.item[z];
  const int nb = t.row[z + 1] - t.row[z];
  const int npairs = score_pairs(nb);
  const int g = local / npairs;
  const int pair = local - g * npairs;
  const int h = g * a.G + hh;
  int ti, tj;
  band_decode(pair, ti, tj);
  const int n_rows = nb * (kBlock / 8);         // strided rows of this sequence
  const int ibase = ti * kRowsA, jbase = tj * kRowsB;
  const size_t tok0 = (size_t)t.tok[z];

  // Loads: per chunk 32 instructions for A (2048 16-byte slots) and 16 for
  // B (1024); wave w issues A instructions w + 8 m (m < 4) and B
  // instructions w + 8 m (m < 2).  Slot s = 64 k + lane sits at LDS row
  // s / 8, position s % 8, and holds logical piece (s % 8) ^ ((row / 2) % 8)
  // of that row.  Rows past the sequence re-read its last row.
  uint32_t voffA[4], voffB[2];
  {
    const uint32_t strideA = (uint32_t)a.Hq * kHeadDim * 2 * 8, strideB = (uint32_t)a.Hkv * kHeadDim * 2 * 8;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int sl = 64 * (wave + 8 * m) + lane, row = sl >> 3, lc = (sl & 7) ^ ((row >> 1) & 7);
      const int rr = (ibase + row < n_rows ? ibase + row : n_rows - 1) - ibase;
      voffA[m] = (uint32_t)rr * strideA + 16 * lc;
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int sl = 64 * (wave + 8 * m) + lane, row = sl >> 3, lc = (sl & 7) ^ ((row >> 1) & 7);
      const int rr = (jbase + row < n_rows ? jbase + row : n_rows - 1) - jbase;
      voffB[m] = (uint32_t)rr * strideB + 16 * lc;
    }
  }
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.q + ((tok0 + 8 * (size_t)ibase) * a.Hq + h) * kHeadDim), (short)0, 0x7fffffff, kScoreBufWord3);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.k + ((tok0 + 8 * (size_t)jbase) * a.Hkv + g) * kHeadDim), (short)0, 0x7fffffff, kScoreBufWord3);
  const uint32_t tokA = (uint32_t)a.Hq * kHeadDim * 2, tokB = (uint32_t)a.Hkv * kHeadDim * 2;
  // chunk c: token t = c / 2 of the stride group (reversed for K), dims 64 (c % 2)
  auto issue = [&](int c, uint16_t *Ad, uint16_t *Bd) __attribute__((always_inline)) {
    const int tt = c >> 1, d2 = (c & 1) * kScoreBK * 2;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void_t *)(Ad + (wave + 8 * m) * 512), 16, voffA[m],
                                               (int)(tt * tokA + d2), 0, 0);
#pragma unroll
    for (int m = 0; m < 2; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void_t *)(Bd + (wave + 8 * m) * 512), 16, voffB[m],
                                               (int)((7 - tt) * tokB + d2), 0, 0);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) acc[mi][nj] = f32x16{};

  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, lg = lane >> 5;
  // fragment rows wm*64 + 32 mi + frow (A) and wn*64 + 32 nj + frow (B): the
  // permutation key (row / 2) % 8 is (frow / 2) % 8 for all of them
  const int swz = (frow >> 1) & 7;
  int poff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) poff[ks] = 8 * ((2 * ks + lg) ^ swz);
  const int rowA = (wm * 64 + frow) * kScoreBK, rowB = (wn * 64 + frow) * kScoreBK;

  auto compute = [&](const uint16_t *As, const uint16_t *Bs) __attribute__((always_inline)) {
    u32x4 fa[2][2], fb[2][2];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) fa[0][mi] = ld16(As + rowA + 32 * mi * kScoreBK + poff[0]);
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) fb[0][nj] = ld16(Bs + rowB + 32 * nj * kScoreBK + poff[0]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) fa[(ks + 1) & 1][mi] = ld16(As + rowA + 32 * mi * kScoreBK + poff[ks + 1]);
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) fb[(ks + 1) & 1][nj] = ld16(Bs + rowB + 32 * nj * kScoreBK + poff[ks + 1]);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj)
          acc[mi][nj] = mfma_bf16_32x32x16(as_bf16x8(fa[ks & 1][mi]), as_bf16x8(fb[ks & 1][nj]), acc[mi][nj]);
    }
  };

  issue(0, A0, B0);
  issue(1, A1, B1);
  score_static_for<kChunks>([&](auto C_) {
    constexpr int c = decltype(C_)::value;
    if constexpr (c + 1 < kChunks) score_wait_vmcnt<6>();   // chunk c+1's six loads may still fly
    else score_wait_vmcnt<0>();
    score_sync();                                          // chunk c everywhere; stage of c-1 free
    if constexpr (c + 2 < kChunks) {
      if constexpr ((c + 2) % 3 == 0) issue(c + 2, A0, B0);
      else if constexpr ((c + 2) % 3 == 1) issue(c + 2, A1, B1);
      else issue(c + 2, A2, B2);
    }
    __builtin_amdgcn_sched_barrier(0);                     // keep the loads ahead of this chunk's MFMAs
    if constexpr (c % 3 == 0) compute(A0, B0);
    else if constexpr (c % 3 == 1) compute(A1, B1);
    else compute(A2, B2);
  });

  // ---- epilogue: causal mask, 16x16 max-pool, scale, bonus
  const bool diag = tj >= 2 * ti;              // some key column of the tile lies past some query row
  const size_t srow0 = ((size_t)h * a.R + t.row[z]) * a.max_nb;
  const float *bon = a.bonus + (size_t)g * a.R + t.row[z];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) {
      const int ib = ibase + wm * 64 + mi * 32;   // strided row base
      const int jb = jbase + wn * 64 + nj * 32;
      const int j = jb + (lane & 31);
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = ib + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float x = acc[mi][nj][r];
        if (diag && j > i) x = -INFINITY;
        if (r < 8) m0 = fmaxf(m0, x); else m1 = fmaxf(m1, x);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        m0 = fmaxf(m0, __shfl_xor(m0, o, 64));
        m1 = fmaxf(m1, __shfl_xor(m1, o, 64));
      }
      m0 = fmaxf(m0, __shfl_xor(m0, 32, 64));
      m1 = fmaxf(m1, __shfl_xor(m1, 32, 64));
      if ((lane & 15) == 0 && lane < 32) {
        const int J = jb / 16 + (lane >> 4);
        const int I0 = ib / 16;
        if (J < nb) {
          if (I0 < nb) a.scores[srow0 + (size_t)I0 * a.max_nb + J] = m0 * a.scale + bon[J];
          if (I0 + 1 < nb) a.scores[srow0 + (size_t)(I0 + 1) * a.max_nb + J] = m1 * a.scale + bon[J];
        }
      }
    }
  }
  const int nt_c = (nb + 7) / 8;
  const int tj_last = 2 * ti + 1 < nt_c - 1 ? 2 * ti + 1 : nt_c - 1;
  if (tj == tj_last) {
    // -inf for the columns this row band never computes: J past its last
    // column band (non-causal) and J >= nb (past the sequence, up to max_nb).
    int jstart = (tj_last + 1) * 8;
    if (jstart > nb) jstart = nb;
    const int width = a.max_nb - jstart;
    for (int e = tid; e < 16 * width; e += 512) {
      const int I = ti * 16 + e / width, J = jstart + e % width;
      if (I < nb) a.scores[srow0 + (size_t)I * a.max_nb + J] = -INFINITY;
    }
  }
}

hipError_t launch_score(const ScoreLaunch &l, const SeqTable &t, int n_items, hipStream_t s) {
  ScoreArgs a;
  a.q = (const __bf16 *)l.q;
  a.k = (const __bf16 *)l.k;
  a.bonus = l.ell;
  a.scores = l.scores;
  a.Hq = l.Hq;
  a.Hkv = l.Hkv;
  a.R = l.R;
  a.max_nb = l.max_nb;
  a.G = l.Hq / l.Hkv;
  a.scale = l.scale;
  hipLaunchKernelGGL(score_kernel, dim3(n_items), dim3(512), 0, s, a, t, n_items);
  return hipGetLastError();
}

}  // namespace stem
