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
//           into the epilogue.  Only the causal triangle of 128x128 strided
//           tiles is launched; scores never touch HBM before pooling.
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
// Workgroup tile: 128 strided query rows x 128 strided key rows (= 8 x 8
// blocks of 16 strided rows), K = s*d = 1024 walked in 16 chunks of 64.
// Row i of the A matrix is Q[tok + i*s + t][h][:] for t = 0..s-1; row j of B
// is K[tok + j*s + (s-1-t)][g][:] (the anti-diagonal pairing).  Chunk c
// covers t = c / 2 and head dims (c % 2) * 64 .. +63, so every lane's load is
// 16 contiguous bytes of one token row.
// Four waves in a 2x2 grid, each 64x64 = 2x2 MFMA 32x32 tiles.
constexpr int kScoreTile = 128;
constexpr int kScoreBK = 64;
constexpr int kLdsRow = kScoreBK + 8;   // 144-byte rows: conflict-free 16 B reads

struct ScoreArgs {
  const __bf16 *q, *k;
  const float *bonus;
  float *scores;
  int32_t Hq, Hkv, R, max_nb, G;
  float scale;
};

__device__ __forceinline__ void tri_decode(int p, int &ti, int &tj) {
  // p = ti*(ti+1)/2 + tj, 0 <= tj <= ti
  int r = (int)((sqrtf(8.f * (float)p + 1.f) - 1.f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= p) ++r;
  while (r * (r + 1) / 2 > p) --r;
  ti = r;
  tj = p - r * (r + 1) / 2;
}

__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a, SeqTable t, int n_items) {
  __shared__ __attribute__((aligned(16))) __bf16 As[2][kScoreTile * kLdsRow];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[2][kScoreTile * kLdsRow];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int item = xcd_item(blockIdx.x, n_items, a.G);
  const int slot = item / a.G, hh = item - slot * a.G;
  // slot -> (sequence, KV head, tile pair); item prefix counts slots
  const int z = seq_of(t.item, t.n, slot);
  const int local = slot - t.item[z];
  const int nb = t.row[z + 1] - t.row[z];
  const int nt = (nb + 7) >> 3;
  const int npairs = nt * (nt + 1) / 2;
  const int g = local / npairs;
  const int pair = local - g * npairs;
  const int h = g * a.G + hh;
  int ti, tj;
  tri_decode(pair, ti, tj);

  const int n_rows = nb * (kBlock / 8);         // strided rows of this sequence
  const size_t tok0 = (size_t)t.tok[z];

  // global -> register staging: thread covers rows (tid>>3) + 32p, 16 B col
  const int lrow = tid >> 3, lcol = tid & 7;
  u32x4 ra[4], rb[4];
  auto load_chunk = [&](int c) {
    const int tt = c >> 1, c0 = (c & 1) * kScoreBK + lcol * 8;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      int i = ti * kScoreTile + lrow + 32 * p;
      int j = tj * kScoreTile + lrow + 32 * p;
      i = i < n_rows ? i : n_rows - 1;
      j = j < n_rows ? j : n_rows - 1;
      const size_t qt = tok0 + (size_t)i * 8 + tt;
      const size_t kt = tok0 + (size_t)j * 8 + (7 - tt);
      ra[p] = ld16(a.q + (qt * a.Hq + h) * kHeadDim + c0);
      rb[p] = ld16(a.k + (kt * a.Hkv + g) * kHeadDim + c0);
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      st16(&As[buf][(lrow + 32 * p) * kLdsRow + lcol * 8], ra[p]);
      st16(&Bs[buf][(lrow + 32 * p) * kLdsRow + lcol * 8], rb[p]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) acc[mi][nj] = f32x16{};

  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  constexpr int kChunks = 8 * kHeadDim / kScoreBK;   // s*d / 64 = 16

  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < kChunks; ++c) {
    const int buf = c & 1;
    if (c + 1 < kChunks) load_chunk(c + 1);
#pragma unroll
    for (int ks = 0; ks < kScoreBK / 16; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        fa[mi] = as_bf16x8(ld16(&As[buf][(wm * 64 + mi * 32 + frow) * kLdsRow + ks * 16 + fk]));
#pragma unroll
      for (int nj = 0; nj < 2; ++nj)
        fb[nj] = as_bf16x8(ld16(&Bs[buf][(wn * 64 + nj * 32 + frow) * kLdsRow + ks * 16 + fk]));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 2; ++nj) acc[mi][nj] = mfma_bf16_32x32x16(fa[mi], fb[nj], acc[mi][nj]);
    }
    if (c + 1 < kChunks) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: causal mask, 16x16 max-pool, scale, bonus
  const bool diag = (ti == tj);
  const size_t srow0 = ((size_t)h * a.R + t.row[z]) * a.max_nb;
  const float *bon = a.bonus + (size_t)g * a.R + t.row[z];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int nj = 0; nj < 2; ++nj) {
      const int ib = ti * kScoreTile + wm * 64 + mi * 32;   // strided row base
      const int jb = tj * kScoreTile + wn * 64 + nj * 32;
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
  if (diag) {
    // -inf for the columns this row band never computes: J beyond the tile
    // (non-causal) and J >= nb (past the sequence, up to max_nb).
    int jstart = (ti + 1) * 8;
    if (jstart > nb) jstart = nb;
    const int width = a.max_nb - jstart;
    for (int e = tid; e < 8 * width; e += 256) {
      const int I = ti * 8 + e / width, J = jstart + e % width;
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
  hipLaunchKernelGGL(score_kernel, dim3(n_items), dim3(256), 0, s, a, t, n_items);
  return hipGetLastError();
}

}  // namespace stem
