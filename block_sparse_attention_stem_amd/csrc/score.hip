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
//           into the epilogue.  Only the causal triangle of 256x256 strided
//           tiles is launched; scores never touch HBM before pooling.
#include <type_traits>
#include <utility>

#include "stem_internal.h"
#include "gfx950_util.h"

namespace stem {

// ------------------------------------------------------------------ vnorm
// One workgroup per (global key block, KV head); 16 lanes per token row
// (16 x 16 B = 256 B = one head vector), 16 rows per pass.
// Both value-norm kernels also zero the scoring kernel's work-queue counters
// (ctr, n_ctr of them), which run after them on the same stream.
__global__ __launch_bounds__(256) void vnorm_kernel(const __bf16 *__restrict__ v,
                                                    float *__restrict__ ell, int Hkv, int R,
                                                    int32_t *__restrict__ ctr, int n_ctr) {
  const int kb = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, sub = tid & 15, rowg = tid >> 4;
  if (kb == 0 && g == 0)
    for (int i = tid; i < n_ctr; i += 256) ctr[i] = 0;
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

// e4m3 V: ||V_t||^2 = vs_J^2 sum_d code_d^2 with vs_J the block's V scale.
// 8 lanes per token row (8 x 16 codes), 32 rows per pass.
__global__ __launch_bounds__(256) void vnorm_fp8_kernel(const uint8_t *__restrict__ v, const float *__restrict__ vsc,
                                                        float *__restrict__ ell, int Hkv, int R,
                                                        int32_t *__restrict__ ctr, int n_ctr) {
  const int kb = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, sub = tid & 7, rowg = tid >> 3;
  if (kb == 0 && g == 0)
    for (int i = tid; i < n_ctr; i += 256) ctr[i] = 0;
  __shared__ float red[32];
  float emax = 0.f;
  for (int t = rowg; t < kBlock; t += 32) {
    const size_t tok = (size_t)kb * kBlock + t;
    const u32x4 raw = ld16(v + (tok * Hkv + g) * kHeadDim + sub * 16);
    float e = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[w], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)raw[w], true);
      e = fmaf(lo[0], lo[0], e);
      e = fmaf(lo[1], lo[1], e);
      e = fmaf(hi[0], hi[0], e);
      e = fmaf(hi[1], hi[1], e);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) e += __shfl_xor(e, o, 64);
    emax = fmaxf(emax, e);
  }
  if (sub == 0) red[rowg] = emax;
  __syncthreads();
  if (tid == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) m = fmaxf(m, red[i]);
    const float vs = vsc[(size_t)kb * Hkv + g];
    ell[(size_t)g * R + kb] = logf(fmaxf(vs * vs * m, 1e-30f));
  }
}

hipError_t launch_vnorm(const ScoreLaunch &a, hipStream_t s) {
  dim3 grid(a.R, a.Hkv);
  if (a.fp8)
    hipLaunchKernelGGL(vnorm_fp8_kernel, grid, dim3(256), 0, s, (const uint8_t *)a.v, a.v_scale, a.ell, a.Hkv, a.R,
                       a.ctr, a.n_ctr);
  else
    hipLaunchKernelGGL(vnorm_kernel, grid, dim3(256), 0, s, (const __bf16 *)a.v, a.ell, a.Hkv, a.R, a.ctr, a.n_ctr);
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
// Workgroup tile: 256 strided query rows x 256 strided key rows (= 16 x 16
// blocks of 16 strided rows), K = s*d = 1024 walked in 32 chunks of 32.
// Row i of the A matrix is Q[tok + i*s + t][h][:] for t = 0..s-1; row j of B
// is K[tok + j*s + (s-1-t)][g][:] (the anti-diagonal pairing).  Chunk c
// covers t = c / 4 and head dims (c % 4) * 32 .. +31: one 64-byte piece of
// one token row per matrix row.
//
// Eight waves (two per SIMD) in a 4 x 2 grid, each 64 x 128 = 2 x 4 MFMA
// 32x32 tiles: a fragment read from LDS feeds two (A) or four (B) MFMAs
// (768 LDS bytes per MFMA).  Chunks arrive by direct-to-LDS buffer loads
// into a ring of four stages (separate LDS arrays, the chunk loop fully
// unrolled), requested four chunks ahead, with one barrier per chunk and no
// staging registers; a chunk's fragments are read into registers while the
// previous chunk's MFMAs run, so LDS latency is never waited on.  LDS rows
// are 64 bytes; a row's 16-byte pieces are stored XOR-permuted by (row / 4)
// % 4, so the fragment reads of an MFMA hit every bank once.  The
// permutation is applied on the global side of the loads (each lane fetches
// the piece that belongs at its fixed LDS slot).
//
// The grid is persistent: one workgroup per CU takes tiles from a work
// queue per XCD (stealing from the other XCDs at the end), and the ring runs
// on across tiles: the last steps of a tile request the first chunks of the
// next one, so a tile's load latency, epilogue and dispatch no longer leave
// the matrix core idle.  Measured on one box with identical scores, against
// one workgroup per tile and against a fixed XCD-local tile list per
// workgroup: 128K layer 6.91 / 7.59 / 7.46 ms, 64K 1.80 / 1.99 / 1.90, the
// fp8 varlen layer 2.90 / 3.34 / 3.08 on bf16 and 1.52 / 2.06 / 1.60 on e4m3
// codes (the fixed list loses to the queue on the CUs and XCDs that run
// slower).  The tile-independent -inf entries of S are written by
// score_fill_kernel.
//
// e4m3 inputs (kFp8): the same tile, rows and loads; a chunk is 64 codes
// (one 64-byte piece of one token row, 16 chunks), one 32x32x64 fp8 MFMA step
// whose 32-byte lane operand is two 16-byte pieces.  Q and K scales are
// constant over a block pair's 16 x 16 strided cells, so they multiply the
// pooled maximum.
constexpr int kTileS = 256;                 // strided rows per tile side
constexpr int kScoreBK = 32;                // K elements per chunk
constexpr int kChunks = 8 * kHeadDim / kScoreBK;   // 32
constexpr int kStages = 4;
constexpr uint32_t kScoreBufWord3 = 0x00020000u;   // raw buffer descriptor word 3 (gfx9 dword access)

struct ScoreArgs {
  const __bf16 *q, *k;
  const float *q_scale, *k_scale;   // kFp8: [R][Hq], [R][Hkv]
  const float *bonus;
  float *scores;
  int32_t Hq, Hkv, R, max_nb, G;
  float scale;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// Tile pair p of a (sequence, head) -> (row band ti, column band tj <= ti),
// p = ti (ti + 1) / 2 + tj.
__device__ __forceinline__ void tri_decode(int p, int &ti, int &tj) {
  int r = (int)((sqrtf(8.f * (float)p + 1.f) - 1.f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= p) ++r;
  while (r * (r + 1) / 2 > p) --r;
  ti = r;
  tj = p - r * (r + 1) / 2;
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

// Cross-lane max-pool on an order-preserving integer image of the floats:
// for non-NaN x, key(x) = bits ^ ((bits >> 31) & 0x7fffffff) orders like x as
// a signed integer and is its own inverse.  Integer max needs no IEEE
// canonicalisation, so each DPP step folds into one v_max_i32.
__device__ __forceinline__ int max_key(float x) {
  const int b = __float_as_int(x);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key_max(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }
template <int kCtrl>
__device__ __forceinline__ int dpp_imax(int k) {
  const int o = __builtin_amdgcn_update_dpp(0, k, kCtrl, 0xF, 0xF, true);
  return k > o ? k : o;
}
// k[n] <- max over its row of 16 lanes (pairs, quads, half-row mirror, row
// mirror), then over lanes l and l ^ 32 (v_permlane32_swap with the value as
// both operands returns both halves' values).  The N chains advance one step
// at a time, so no DPP read waits on the write just before it.
template <int N>
__device__ __forceinline__ void key_max_rows_and_halves(int (&k)[N]) {
#pragma unroll
  for (int n = 0; n < N; ++n) k[n] = dpp_imax<0xB1>(k[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) k[n] = dpp_imax<0x4E>(k[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) k[n] = dpp_imax<0x141>(k[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) k[n] = dpp_imax<0x140>(k[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)k[n], (unsigned)k[n], false, false);
    const int a = (int)r[0], b = (int)r[1];
    k[n] = a > b ? a : b;
  }
}

// Tile of a work item: sequence z of the launch, KV head g, query head h,
// row band ti and column band tj <= ti, and the sequence's block count nb.
struct ScoreTile {
  int z, g, h, ti, tj, nb;
};
// Decoded without loops: the persistent kernel decodes its next tile in the
// middle of the current one, and an inner loop there makes the register
// allocator spill the fragments and accumulators live across it.
__device__ __forceinline__ ScoreTile score_tile(const ScoreArgs &a, const SeqTable &t, int item) {
  ScoreTile T;
  const int slot = item / a.G, hh = item - slot * a.G;
  // largest z < n with item[z] <= slot (item[] is non-decreasing, item[0] = 0
  // <= slot): binary lifting over the kMaxSeqsPerLaunch = 64 entries
  int z = 0;
#pragma unroll
  for (int step = kMaxSeqsPerLaunch / 2; step >= 1; step >>= 1) {
    const int mid = z + step;
    z = (mid < t.n) & (t.item[mid] <= slot) ? mid : z;
  }
  T.z = z;
  const int local = slot - t.item[z];
  T.nb = t.row[z + 1] - t.row[z];
  const int npairs = score_pairs(T.nb);
  T.g = local / npairs;
  T.h = T.g * a.G + hh;
  // row band r of pair p: r (r + 1) / 2 <= p < (r + 1) (r + 2) / 2; the fp32
  // square-root estimate is off by at most one for p < 2^24
  const int p = local - T.g * npairs;
  int r = (int)((sqrtf(8.f * (float)p + 1.f) - 1.f) * 0.5f);
  r = (r + 1) * (r + 2) / 2 <= p ? r + 1 : r;
  r = r * (r + 1) / 2 > p ? r - 1 : r;
  T.ti = r;
  T.tj = p - r * (r + 1) / 2;
  return T;
}

typedef const __attribute__((address_space(4))) float score_cfloat;   // scalar (s_load) reads

template <bool kFp8>
__global__ __launch_bounds__(512, 1) void score_kernel(ScoreArgs a, SeqTable t, int n_items, int32_t *ctr) {
  constexpr int kEsz = kFp8 ? 1 : 2;                      // bytes per element
  constexpr int kNChunks = kFp8 ? kChunks / 2 : kChunks;  // 64 codes or 32 bf16 per chunk
  constexpr int kStores = 16;                             // epilogue stores per wave
  __shared__ __attribute__((aligned(1024))) uint16_t A0[kTileS * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t A1[kTileS * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t A2[kTileS * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t A3[kTileS * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t B0[kTileS * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t B1[kTileS * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t B2[kTileS * kScoreBK];
  __shared__ __attribute__((aligned(1024))) uint16_t B3[kTileS * kScoreBK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Loads: per chunk 16 instructions for A (1024 16-byte slots) and 16 for
  // B; wave w issues A and B instructions w + 8 m (m < 2).  Slot s = 64 k +
  // lane sits at LDS row s / 4, position s % 4, and holds logical piece
  // (s % 4) ^ ((row / 4) % 4) of that row.  Rows past the sequence re-read
  // its last row.  set_loads points the offsets and descriptors at a tile.
  const uint32_t strideA = (uint32_t)a.Hq * kHeadDim * kEsz * 8, strideB = (uint32_t)a.Hkv * kHeadDim * kEsz * 8;
  const uint32_t tokA = (uint32_t)a.Hq * kHeadDim * kEsz, tokB = (uint32_t)a.Hkv * kHeadDim * kEsz;
  uint32_t voffA[2], voffB[2];
  __amdgpu_buffer_rsrc_t rA, rB;
  auto set_loads = [&](const ScoreTile &T, bool live) __attribute__((always_inline)) {
    const int n_rows = T.nb * (kBlock / 8);       // strided rows of this sequence
    const int ibase = T.ti * kTileS, jbase = T.tj * kTileS;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int sl = 64 * (wave + 8 * m) + lane, row = sl >> 2, lc = (sl & 3) ^ ((row >> 2) & 3);
      const int ra = (ibase + row < n_rows ? ibase + row : n_rows - 1) - ibase;
      const int rb = (jbase + row < n_rows ? jbase + row : n_rows - 1) - jbase;
      voffA[m] = (uint32_t)ra * strideA + 16 * lc;
      voffB[m] = (uint32_t)rb * strideB + 16 * lc;
    }
    const size_t tok0 = (size_t)t.tok[T.z];
    rA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)a.q + ((tok0 + 8 * (size_t)ibase) * a.Hq + T.h) * kHeadDim * kEsz), (short)0,
        live ? 0x7fffffff : 0, kScoreBufWord3);
    rB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)((const char *)a.k + ((tok0 + 8 * (size_t)jbase) * a.Hkv + T.g) * kHeadDim * kEsz), (short)0,
        live ? 0x7fffffff : 0, kScoreBufWord3);
  };
  // chunk c: token t = c / 4 of the stride group (reversed for K), dims 32 (c % 4);
  // kFp8: token t = c / 2, codes 64 (c % 2)
  // wl, tA and tB are wave, tokA and tokB, re-declared opaque at the top of
  // every tile (an empty asm): otherwise the compiler hoists each chunk's
  // LDS destinations and scalar offsets, loop-invariant, out of the tile
  // loop, and holding those ~80 values across it overflows the SGPRs.
  int wl = wave;
  uint32_t tA = tokA, tB = tokB;
  auto issue = [&](int c, uint16_t *Ad, uint16_t *Bd) __attribute__((always_inline)) {
    const int tt = kFp8 ? c >> 1 : c >> 2, d2 = (kFp8 ? (c & 1) : (c & 3)) * 64;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void_t *)(Ad + (wl + 8 * m) * 512), 16, voffA[m],
                                               (int)(tt * tA + d2), 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void_t *)(Bd + (wl + 8 * m) * 512), 16, voffB[m],
                                               (int)((7 - tt) * tB + d2), 0, 0);
    }
  };

  f32x16 acc[2][4];

  const int frow = lane & 31, lg = lane >> 5;
  // fragment rows wm*64 + 32 mi + frow (A) and wn*128 + 32 nj + frow (B):
  // the permutation key (row / 4) % 4 is (frow / 4) % 4 for all of them
  const int swz = (frow >> 2) & 3;
  // 16-byte piece read for index x: bf16, k-step x; e4m3, half x of the lane's 32 bytes
  int poff[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) poff[x] = 8 * ((kFp8 ? 2 * lg + x : 2 * x + lg) ^ swz);
  const int rowA = (wm * 64 + frow) * kScoreBK, rowB = (wn * 128 + frow) * kScoreBK;

  // Fragments of a chunk: 2 k-steps x (2 A + 4 B) 16-byte reads (bf16), or
  // 2 A + 4 B operands of 32 bytes, each two 16-byte reads (e4m3).
  typedef u32x4 Frags16[2][6];
  typedef i32x8 Frags8[6];
  using Frags = std::conditional_t<kFp8, Frags8, Frags16>;
  auto read_frags = [&](Frags &f, const uint16_t *As, const uint16_t *Bs) __attribute__((always_inline)) {
    if constexpr (kFp8) {
      auto ld32 = [&](const uint16_t *row) __attribute__((always_inline)) {
        const u32x4 lo = ld16(row + poff[0]), hi = ld16(row + poff[1]);
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      };
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) f[mi] = ld32(As + rowA + 32 * mi * kScoreBK);
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) f[2 + nj] = ld32(Bs + rowB + 32 * nj * kScoreBK);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) f[ks][mi] = ld16(As + rowA + 32 * mi * kScoreBK + poff[ks]);
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) f[ks][2 + nj] = ld16(Bs + rowB + 32 * nj * kScoreBK + poff[ks]);
      }
    }
  };
  auto mfmas = [&](const Frags &f) __attribute__((always_inline)) {
    if constexpr (kFp8) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = mfma_fp8_32x32x64(f[mi], f[2 + nj], acc[mi][nj]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int nj = 0; nj < 4; ++nj)
            acc[mi][nj] = mfma_bf16_32x32x16(as_bf16x8(f[ks][mi]), as_bf16x8(f[ks][2 + nj]), acc[mi][nj]);
    }
  };
  auto stage_issue = [&](auto S_, int c) __attribute__((always_inline)) {
    constexpr int st = decltype(S_)::value;
    if constexpr (st == 0) issue(c, A0, B0);
    else if constexpr (st == 1) issue(c, A1, B1);
    else if constexpr (st == 2) issue(c, A2, B2);
    else issue(c, A3, B3);
  };
  auto stage_read = [&](auto S_, Frags &f) __attribute__((always_inline)) {
    constexpr int st = decltype(S_)::value;
    if constexpr (st == 0) read_frags(f, A0, B0);
    else if constexpr (st == 1) read_frags(f, A1, B1);
    else if constexpr (st == 2) read_frags(f, A2, B2);
    else read_frags(f, A3, B3);
  };

  // Epilogue operands, read through scalar loads during the tile (their
  // wait is the lgkmcnt(0) of a later barrier): this wave's block columns
  // J = 16 tj + 8 wn + e (e < 8) and rows I = 16 ti + 4 wm + e (e < 4),
  // clamped into the sequence (values of clamped entries are never stored).
  float bon_s[8], ksc_s[8], qsc_s[4];
  auto load_epilogue = [&](const ScoreTile &T) __attribute__((always_inline)) {
    const int r0 = t.row[T.z], j0 = 16 * T.tj + 8 * wn, i0 = 16 * T.ti + 4 * wm;
    score_cfloat *bon = (score_cfloat *)a.bonus + (size_t)T.g * a.R + r0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int J = j0 + e < T.nb ? j0 + e : T.nb - 1;
      bon_s[e] = bon[J];
      if constexpr (kFp8) ksc_s[e] = ((score_cfloat *)a.k_scale)[(size_t)(r0 + J) * a.Hkv + T.g];
    }
    if constexpr (kFp8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int I = i0 + e < T.nb ? i0 + e : T.nb - 1;
        qsc_s[e] = ((score_cfloat *)a.q_scale)[(size_t)(r0 + I) * a.Hq + T.h];
      }
    }
  };

  // Causal mask, 16x16 max-pool, scale and bonus; then exactly kStores
  // buffer stores per wave into the tile's row band of S, whatever the
  // tile: a lane with nothing to store (or a block past the sequence) gives
  // an offset beyond the descriptor's range, which drops its store.  The
  // fixed count keeps the vmcnt arithmetic of the next tile's waits exact.
  auto epilogue = [&](const ScoreTile &T) __attribute__((always_inline)) {
    if (T.ti == T.tj) {
      // The strided causal mask j <= i (only the diagonal tile crosses it).
      // There ibase = jbase, and MFMA tile (mi, nj) of this wave starts
      // off = 128 wn + 32 nj - 64 wm - 32 mi columns right of its first
      // row (a multiple of 32, the same for the whole wave): off > 0 is
      // wholly above the diagonal, off < 0 wholly below, and off = 0 holds
      // it, with j - i = d - (8 (r / 4) + r % 4) for element r of the lane.
      // d is formed from an opaque copy of the lane index, so that the
      // compiler neither hoists its loop-invariant compares out of the tile
      // loop nor keeps d itself live (spilled) across it.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int d = (ln & 31) - 4 * (ln >> 5);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int nj = 0; nj < 4; ++nj) {
          const int off = 128 * wn + 32 * nj - 64 * wm - 32 * mi;
          if (off > 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mi][nj][r] = -INFINITY;
          } else if (off == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (d > 8 * (r >> 2) + (r & 3)) acc[mi][nj][r] = -INFINITY;
          }
        }
    }
    // per lane: the max of its 8 rows of each 16-row half, then across lanes
    int key[16];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) {
        float m0 = acc[mi][nj][0], m1 = acc[mi][nj][8];
#pragma unroll
        for (int r = 1; r < 8; ++r) {
          m0 = fmaxf(m0, acc[mi][nj][r]);
          m1 = fmaxf(m1, acc[mi][nj][8 + r]);
        }
        key[8 * mi + 2 * nj] = max_key(m0);
        key[8 * mi + 2 * nj + 1] = max_key(m1);
      }
    key_max_rows_and_halves(key);
    const int rows = T.nb - 16 * T.ti < 16 ? T.nb - 16 * T.ti : 16;
    const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.scores + ((size_t)T.h * a.R + t.row[T.z] + 16 * T.ti) * a.max_nb), (short)0,
        rows * a.max_nb * 4, kScoreBufWord3);
    const int hl = (lane >> 4) & 1;
    const bool writer = (lane & 15) == 0 && lane < 32;
    // x1 for lanes 16-31, x0 for the others, as a bit select: written as
    // hl ? x[1] : x[0] the compiler turns it into x[hl], an indexed read
    // of a scratch copy of the array
    const uint32_t hmask = 0u - (uint32_t)hl;
    auto pick = [&](float x0, float x1) __attribute__((always_inline)) {
      return __uint_as_float((__float_as_uint(x1) & hmask) | (__float_as_uint(x0) & ~hmask));
    };
    __builtin_amdgcn_sched_barrier(0);    // the stores stay between this tile's loads and the next tile's
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) {
        const int Jl = 16 * T.tj + 8 * wn + 2 * nj + hl;   // block column in the sequence
        const int Il = 4 * wm + 2 * mi;                      // block row within the band
        const float m0 = key_max(key[8 * mi + 2 * nj]), m1 = key_max(key[8 * mi + 2 * nj + 1]);
        const float bn = pick(bon_s[2 * nj], bon_s[2 * nj + 1]);
        float v0, v1;
        if constexpr (kFp8) {
          // scores of the dequantised values: raw max x q scale of row I x k scale of J
          const float sk = a.scale * pick(ksc_s[2 * nj], ksc_s[2 * nj + 1]);
          v0 = m0 * (sk * qsc_s[2 * mi]) + bn;
          v1 = m1 * (sk * qsc_s[2 * mi + 1]) + bn;
        } else {
          v0 = m0 * a.scale + bn;
          v1 = m1 * a.scale + bn;
        }
        const bool ok = writer && Jl < T.nb;
        const uint32_t o0 = ok ? (uint32_t)(Il * a.max_nb + Jl) * 4u : 0x80000000u;
        const uint32_t o1 = ok ? (uint32_t)((Il + 1) * a.max_nb + Jl) * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v0), rS, (int)o0, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v1), rS, (int)o1, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Pipeline.  Step c of a tile: wait for chunk c+1, barrier (chunk c's
  // fragments, read in step c-1, are out of its stage everywhere), issue the
  // loads of chunk c+4 into that stage, then run chunk c's MFMAs from
  // registers with the fragment reads of chunk c+1 between them.  The grid
  // is persistent: in the last steps of a tile the chunks "c+4" are chunks
  // 0-2 of the workgroup's next tile, so its loads fly during the end of
  // this tile and its epilogue; chunk 3 follows at the next tile's first
  // barrier.  In-flight loads per wave at each wait (4 per chunk, in issue
  // order with the 16 epilogue stores): the chunks after the awaited one,
  // plus the stores while they sit behind it (the first tile is preceded by
  // 16 stores to an empty range, so every tile sees the same sequence).
  // Work queue (as for the attention kernels): XCD x = blockIdx % 8 owns
  // the contiguous items [x per, (x + 1) per), handed out in order by the
  // counter ctr[x] (zeroed by the value-norm kernel), so an XCD's
  // workgroups hold neighbouring tiles of one KV group in its L2 at any
  // time; once its items are gone a workgroup takes items of the other
  // XCDs.  Thread 0 claims one tile ahead of the decode: at the top of tile
  // n it turns the counter value fetched at tile n-1 into the item of tile
  // n+2 (an LDS slot by parity) and fetches the next value, so no atomic
  // result is waited for inside the tile.
  __shared__ int32_t q_slot[3];
  const int per = (n_items + 7) >> 3, xcd = blockIdx.x & 7;
  auto claim = [&](int i) {              // thread 0 only; -1 when every item is taken
    const int lo = xcd * per, hi = lo + per < n_items ? lo + per : n_items;
    if (lo + i < hi) return lo + i;
    for (int k = 1; k < 8; ++k) {
      const int x = (xcd + k) & 7, xl = x * per, xh = xl + per < n_items ? xl + per : n_items;
      if (xl >= xh || __hip_atomic_load(&ctr[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= xh - xl) continue;
      const int y = atomicAdd(&ctr[x], 1);
      if (xl + y < xh) return xl + y;
    }
    return -1;
  };
  int pending = 0;
  if (tid == 0) {
    q_slot[2] = claim(atomicAdd(&ctr[xcd], 1));
    q_slot[0] = claim(atomicAdd(&ctr[xcd], 1));
    pending = atomicAdd(&ctr[xcd], 1);
  }
  __syncthreads();
  const int first = __builtin_amdgcn_readfirstlane(q_slot[2]);
  if (first < 0) return;
  ScoreTile T = score_tile(a, t, first);
  set_loads(T, true);
  stage_issue(std::integral_constant<int, 0>{}, 0);
  stage_issue(std::integral_constant<int, 1>{}, 1);
  stage_issue(std::integral_constant<int, 2>{}, 2);
  {
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(a.scores, (short)0, 0, kScoreBufWord3);
    __builtin_amdgcn_sched_barrier(0);    // the counts need the loads before the stores
#pragma unroll
    for (int i = 0; i < kStores; ++i)   // offsets 4 KB apart: never merged into wider stores
      __builtin_amdgcn_raw_buffer_store_b32(0u, none, 4096 * i, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  Frags fr[2];
  int j = 0;
  while (true) {
    // the next tile is decoded here, where no accumulator or fragment is
    // live (decoded mid-tile, its temporaries pushed the fp8 kernel past
    // 256 VGPRs)
    const int nxt = __builtin_amdgcn_readfirstlane(q_slot[j & 1]);
    const bool has_next = nxt >= 0;
    if (tid == 0) {
      const int nn = has_next ? claim(pending) : -1;
      q_slot[(j + 1) & 1] = nn;
      if (nn >= 0) pending = atomicAdd(&ctr[xcd], 1);
    }
    const ScoreTile Tn = has_next ? score_tile(a, t, nxt) : T;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nj = 0; nj < 4; ++nj) acc[mi][nj] = f32x16{};
    asm volatile("" : "+s"(wl), "+s"(tA), "+s"(tB));
    score_wait_vmcnt<8 + kStores>();              // chunk 0 (chunks 1, 2 and the stores may fly)
    score_sync();
    stage_issue(std::integral_constant<int, 3>{}, 3);
    stage_read(std::integral_constant<int, 0>{}, fr[0]);
    score_static_for<kNChunks>([&](auto C_) {
      constexpr int c = decltype(C_)::value;
      if constexpr (c + 1 < kNChunks) {
        if constexpr (c < 2) score_wait_vmcnt<8 + kStores>();   // the stores sit behind chunk c+1
        else score_wait_vmcnt<8>();
        score_sync();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (c + kStages < kNChunks) {
          stage_issue(std::integral_constant<int, c % kStages>{}, c + kStages);
          if constexpr (c + kStages + 1 == kNChunks) {
            // this tile's last load is out: point the loads at the next tile
            // (after the last tile, at an empty range: the loads still go,
            // read nothing and fill stages that are not read again, so the
            // counts above hold for every tile)
            set_loads(Tn, has_next);
          }
        } else {
          stage_issue(std::integral_constant<int, c % kStages>{}, c + kStages - kNChunks);
        }
        if constexpr (c == 4) load_epilogue(T);
        stage_read(std::integral_constant<int, (c + 1) % kStages>{}, fr[(c + 1) & 1]);
        mfmas(fr[c & 1]);
        // The loads and fragment reads go between the MFMAs (none depends on
        // them): per group of four MFMAs, one fragment read after each of the
        // first three and one tile load after the first.  Issued as a burst
        // before the MFMAs they held both waves of a SIMD off the matrix core
        // at the start of every step.
        if constexpr (kFp8) {
          // 8 MFMAs, 12 fragment reads, 4 loads: per pair of MFMAs, three reads and a load
          score_static_for<4>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          });
        } else {
          score_static_for<4>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // buffer load
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          });
        }
        __builtin_amdgcn_sched_barrier(0);
      } else {
        __builtin_amdgcn_sched_barrier(0);
        mfmas(fr[c & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    epilogue(T);
    if (!has_next) {
      score_wait_vmcnt<0>();       // no load into the LDS may outlive the workgroup
      break;
    }
    T = Tn;
    ++j;
  }
}

// Entries of S no tile writes: for block row I of a sequence with nb blocks,
// J in [min(nb, 16 (I / 16 + 1)), max_nb), i.e. past the row's diagonal tile
// (non-causal) or past the sequence; they are -inf.  One workgroup per
// (block row, query head) of the launch.
__global__ __launch_bounds__(256) void score_fill_kernel(float *__restrict__ scores, SeqTable t, int R,
                                                         int max_nb) {
  const int r = t.row[0] + blockIdx.x, h = blockIdx.y;
  const int z = seq_of(t.row, t.n, r);
  const int I = r - t.row[z], nb = t.row[z + 1] - t.row[z];
  int j0 = 16 * (I / 16 + 1);
  if (j0 > nb) j0 = nb;
  float *row = scores + ((size_t)h * R + r) * max_nb;
  for (int J = j0 + (int)threadIdx.x; J < max_nb; J += 256) row[J] = -INFINITY;
}

size_t score_workspace_ctr_offset(int Hkv, int R) { return ((size_t)Hkv * R * sizeof(float) + 255) / 256 * 256; }
size_t score_workspace_bytes(int Hkv, int R, int num_seqs) {
  const size_t launches = (size_t)(num_seqs + kMaxSeqsPerLaunch - 1) / kMaxSeqsPerLaunch;
  return score_workspace_ctr_offset(Hkv, R) + (launches * 8 * sizeof(int32_t) + 255) / 256 * 256;
}

// CUs of the stream's device (256 if the query fails).
static int score_device_cus(hipStream_t s) {
  int dev = 0;
  if (s) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(s, &d) == hipSuccess) dev = (int)d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    dev = 0;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  return cus;
}

hipError_t launch_score(const ScoreLaunch &l, const SeqTable &t, int n_items, int launch_index, hipStream_t s) {
  ScoreArgs a;
  a.q = (const __bf16 *)l.q;
  a.k = (const __bf16 *)l.k;
  a.q_scale = l.q_scale;
  a.k_scale = l.k_scale;
  a.bonus = l.ell;
  a.scores = l.scores;
  a.Hq = l.Hq;
  a.Hkv = l.Hkv;
  a.R = l.R;
  a.max_nb = l.max_nb;
  a.G = l.Hq / l.Hkv;
  a.scale = l.scale;
  const int rows = t.row[t.n] - t.row[0];
  hipLaunchKernelGGL(score_fill_kernel, dim3(rows, l.Hq), dim3(256), 0, s, l.scores, t, l.R, l.max_nb);
  // persistent: one workgroup per CU, at most one per item
  const int cus = score_device_cus(s);
  const int grid = n_items < cus ? n_items : cus;
  int32_t *ctr = l.ctr + 8 * launch_index;
  if (l.fp8) hipLaunchKernelGGL(score_kernel<true>, dim3(grid), dim3(512), 0, s, a, t, n_items, ctr);
  else hipLaunchKernelGGL(score_kernel<false>, dim3(grid), dim3(512), 0, s, a, t, n_items, ctr);
  return hipGetLastError();
}

}  // namespace stem
