// Stage 3 - causal block-sparse flash attention on gfx950 (and the dense
// baseline, which is the same tile loop over every causal block).
//
// AngelSlim doc "Stem: Rethinking Causal Information Flow in Sparse
// Attention" §2.3: exact attention on the top-k blocks only (bf16 dense and
// fp8 block-sparse prefill, varlen); youleyou HPC-BSA article §三.3.1: a
// skipped block is equivalent to -inf scores, so online softmax over just the
// listed blocks is exact.
//
// One workgroup (4 waves) per (query head h, query block I): 128 queries,
// 32 per wave.  Everything is computed transposed so that a query lives on a
// lane: S^T = K Q^T (A = K rows from LDS, B = the wave's Q held in
// registers), then O^T += V^T P^T (A = V^T rows from LDS, B = P^T straight
// from the S^T accumulators).  With the 32x32 MFMA output layout, lane l then
// owns query l % 32 for every accumulator, so the online-softmax row max is
// one cross-half exchange and the O rescale is a per-lane scalar.
// The P^T operand is taken from the accumulators as they lie; the matching
// key permutation is applied once, when V is transposed into LDS.
// K/V of the next listed block are fetched into registers while the current
// block is computed (the list is read one entry ahead), so the inner loop
// never tests a block: it only walks the compact list.
#include "stem_internal.h"
#include "gfx950_util.h"

namespace stem {

struct AttnItem {
  int h, g, r, z, I;
};

// Rows are walked from the last (longest causal prefix) to the first; the
// G heads of a KV group share an XCD (see xcd_item).
__device__ __forceinline__ AttnItem decode_attn(const AttnLaunch &a, const SeqTable &t, int rows) {
  const int G = a.Hq / a.Hkv;
  const int n_items = rows * a.Hq;
  const int item = xcd_item(blockIdx.x, n_items, G);
  const int slot = item / G, hh = item - slot * G;
  AttnItem w;
  w.g = slot / rows;
  const int rr = slot - w.g * rows;
  w.h = w.g * G + hh;
  w.r = t.row[0] + (rows - 1 - rr);
  w.z = seq_of(t.row, t.n, w.r);
  w.I = w.r - t.row[w.z];
  return w;
}

// ===================================================================== bf16
constexpr int kRowB = kHeadDim + 8;   // LDS row of 136 bf16 (272 B): conflict-free 16 B reads

// Position of key group kg (4 consecutive keys) inside a transposed V row,
// so that lane group x reads keys {16c + 8j + 4x + r} as 8 contiguous
// elements 16c + 8x + 4j + r (j, r < 4): this is exactly the key set the S^T
// accumulator of lane group x holds for PV step c.
__device__ __forceinline__ int vpos_bf16(int kg) {
  const int q = kg & 3;
  return 16 * (kg >> 2) + 4 * (2 * (q & 1) + (q >> 1));
}

template <bool kSparse>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnLaunch a, SeqTable t, int rows) {
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kBlock * kRowB];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHeadDim * kRowB];   // fp16 V^T

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 5, l32 = lane & 31;
  const AttnItem w = decode_attn(a, t, rows);
  const __bf16 *qp = (const __bf16 *)a.q, *kp = (const __bf16 *)a.k, *vp = (const __bf16 *)a.v;
  __bf16 *op = (__bf16 *)a.out;

  const size_t ztok = (size_t)t.tok[w.z];
  const size_t qtok0 = ztok + (size_t)w.I * kBlock;
  const int qloc = wave * 32 + l32;
  const size_t qtok = qtok0 + qloc;
  const int32_t *list = kSparse ? a.idx + ((size_t)w.h * a.R + w.r) * a.k_cap : nullptr;
  // A list is trusted to be ascending in [0, I]; counts and ids are still
  // clamped so that a malformed list can never address outside the sequence.
  int n_blk = kSparse ? a.cnt[(size_t)w.h * a.R + w.r] : w.I + 1;
  if (kSparse && n_blk > a.k_cap) n_blk = a.k_cap;
  __bf16 *orow = op + (qtok * a.Hq + w.h) * kHeadDim;

  if (n_blk <= 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) st8(orow + 32 * u + 8 * jj + 4 * lg, u32x2{0u, 0u});
    if (a.lse && lg == 0) a.lse[(size_t)w.h * a.T + qtok] = -INFINITY;
    return;
  }

  // Q as the B operand: query qloc, head dims 16 ks + 8 lg .. +7
  bf16x8 qf[8];
  {
    const __bf16 *qrow = qp + (qtok * a.Hq + w.h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
  }

  // staging maps.  K: rows (tid >> 4) + 16 p, 16 B column tid & 15.
  // V: head-dim chunk dc (8 dims), key groups kg0 and kg0 + 16 (4 keys each).
  const int krow = tid >> 4, kcol = tid & 15;
  const int dc = 4 * wave + (lane >> 4), kg0 = lane & 15;
  u32x4 kreg[8], vreg[8];
  auto load_k = [&](int J) {
    const __bf16 *src = kp + ((ztok + (size_t)J * kBlock + krow) * a.Hkv + w.g) * kHeadDim + 8 * kcol;
    const size_t step = (size_t)16 * a.Hkv * kHeadDim;
#pragma unroll
    for (int p = 0; p < 8; ++p) kreg[p] = ld16(src + p * step);
  };
  auto store_k = [&]() {
#pragma unroll
    for (int p = 0; p < 8; ++p) st16(&Ks[(krow + 16 * p) * kRowB + 8 * kcol], kreg[p]);
  };
  auto load_v = [&](int J) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int kg = kg0 + 16 * p;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        vreg[4 * p + e] = ld16(vp + ((ztok + (size_t)J * kBlock + 4 * kg + e) * a.Hkv + w.g) * kHeadDim + 8 * dc);
    }
  };
  // V goes to LDS transposed and converted to fp16 (exact for bf16 values in
  // fp16's range), so that P can be rounded to fp16 rather than bf16 for the
  // P.V product: 11 instead of 8 significant bits on every weight.
  auto store_v = [&]() {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int pos = vpos_bf16(kg0 + 16 * p);
      u32x4 hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int x = 0; x < 4; ++x) hv[e][x] = bf16x2_to_f16x2(vreg[4 * p + e][x]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = perm_b32(hv[1][i >> 1], hv[0][i >> 1], sel);
        const uint32_t hi = perm_b32(hv[3][i >> 1], hv[2][i >> 1], sel);
        st8(&Vt[(8 * dc + i) * kRowB + pos], u32x2{lo, hi});
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};

  auto clampJ = [&](int x) { return x < 0 ? 0 : (x > w.I ? w.I : x); };
  int J = kSparse ? clampJ(list[0]) : 0;
  load_k(J);
  load_v(J);
  store_k();
  store_v();
  __syncthreads();

  for (int b = 0; b < n_blk; ++b) {
    const bool more = b + 1 < n_blk;
    const int Jn = more ? (kSparse ? clampJ(list[b + 1]) : b + 1) : 0;
    if (more) load_k(Jn);

    // ---- S^T = K Q^T
    f32x16 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x16{};
      const __bf16 *kr = &Ks[(32 * tt + l32) * kRowB + 8 * lg];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s[tt] = mfma_bf16_32x32x16(as_bf16x8(ld16(kr + 16 * ks)), qf[ks], s[tt]);
    }

    // ---- online softmax (base 2), causal mask on the diagonal block
    const bool diag = (J == w.I);
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[tt][i] * a.scale_log2;
        if (diag) {
          const int key = 32 * tt + 8 * (i >> 2) + 4 * lg + (i & 3);
          if (key > qloc) x = -INFINITY;
        }
        s[tt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = wave_max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[tt][i] - m_new);
        s[tt][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[u][i] *= alpha;
    }
    f16x8 pk[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int tt = c >> 1, j0 = 2 * (c & 1);
      u32x4 v4;
      v4[0] = pack_f16x2(s[tt][4 * j0 + 0], s[tt][4 * j0 + 1]);
      v4[1] = pack_f16x2(s[tt][4 * j0 + 2], s[tt][4 * j0 + 3]);
      v4[2] = pack_f16x2(s[tt][4 * j0 + 4], s[tt][4 * j0 + 5]);
      v4[3] = pack_f16x2(s[tt][4 * j0 + 6], s[tt][4 * j0 + 7]);
      pk[c] = as_f16x8(v4);
    }
    if (more) load_v(Jn);
    __syncthreads();                 // every wave is done reading Ks
    if (more) store_k();

    // ---- O^T += V^T P^T
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint16_t *vr = &Vt[(32 * u + l32) * kRowB + 8 * lg];
#pragma unroll
      for (int c = 0; c < 8; ++c) o[u] = mfma_f16_32x32x16(as_f16x8(ld16(vr + 16 * c)), pk[c], o[u]);
    }
    __syncthreads();                 // every wave is done reading Vt; Ks is written
    if (more) store_v();
    J = Jn;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 v2;
      v2[0] = pack_bf16x2(o[u][4 * jj + 0] * inv, o[u][4 * jj + 1] * inv);
      v2[1] = pack_bf16x2(o[u][4 * jj + 2] * inv, o[u][4 * jj + 3] * inv);
      st8(orow + 32 * u + 8 * jj + 4 * lg, v2);
    }
  if (a.lse && lg == 0)
    a.lse[(size_t)w.h * a.T + qtok] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
}

// ====================================================================== fp8
// Same structure with e4m3fn operands and the 32x32x64 fp8 MFMA: Q.K^T in two
// K=64 steps per key tile, P quantised to e4m3 as p * 2^8 (p <= 1, so the
// largest code is 256 < 448 and fewer small weights flush to zero), PV in
// two K=64 steps per head-dim tile.  Per-block scales: the q and k scales
// fold into the score scale of the block; the v scale of block J is applied
// by keeping O in units of the current block's v scale (one multiply merged
// with the online-softmax rescale).
constexpr int kRow8 = kHeadDim + 16;  // LDS row of 144 bytes

// Position (bytes) of key group kg inside a transposed V row: lane group x
// reads 32 contiguous bytes for PV step c', holding keys 64c' + 32a + 8j +
// 4x + r at byte 32x + 16a + 4j + r (the S^T accumulator order).
__device__ __forceinline__ int vpos_fp8(int kg) {
  const int q = kg & 15;
  return 64 * (kg >> 4) + 4 * (8 * (q & 1) + 4 * (q >> 3) + ((q >> 1) & 3));
}

__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <bool kSparse>
__global__ __launch_bounds__(256) void attn_fp8_kernel(AttnLaunch a, SeqTable t, int rows) {
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kBlock * kRow8];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[kHeadDim * kRow8];
  __shared__ __attribute__((aligned(16))) uint16_t Vh[kHeadDim * kRowB];   // fp16 V^T, diagonal block

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 5, l32 = lane & 31;
  const AttnItem w = decode_attn(a, t, rows);
  const uint8_t *qp = (const uint8_t *)a.q, *kp = (const uint8_t *)a.k, *vp = (const uint8_t *)a.v;
  __bf16 *op = (__bf16 *)a.out;

  const size_t ztok = (size_t)t.tok[w.z];
  const int zrow = t.row[w.z];
  const size_t qtok0 = ztok + (size_t)w.I * kBlock;
  const int qloc = wave * 32 + l32;
  const size_t qtok = qtok0 + qloc;
  const int32_t *list = kSparse ? a.idx + ((size_t)w.h * a.R + w.r) * a.k_cap : nullptr;
  // A list is trusted to be ascending in [0, I]; counts and ids are still
  // clamped so that a malformed list can never address outside the sequence.
  int n_blk = kSparse ? a.cnt[(size_t)w.h * a.R + w.r] : w.I + 1;
  if (kSparse && n_blk > a.k_cap) n_blk = a.k_cap;
  __bf16 *orow = op + (qtok * a.Hq + w.h) * kHeadDim;

  if (n_blk <= 0) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) st8(orow + 32 * u + 8 * jj + 4 * lg, u32x2{0u, 0u});
    if (a.lse && lg == 0) a.lse[(size_t)w.h * a.T + qtok] = -INFINITY;
    return;
  }

  i32x8 qf[2];
  {
    const uint8_t *qrow = qp + (qtok * a.Hq + w.h) * kHeadDim + 32 * lg;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 lo = ld16(qrow + 64 * ks), hi = ld16(qrow + 64 * ks + 16);
      qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }
  const float qs = a.q_scale[(size_t)w.r * a.Hq + w.h] * a.scale_log2;

  const int krow = tid >> 3, kcol = tid & 7;
  const int kg = lane & 31, dc = (lane >> 5) + 2 * wave;   // V: 4 keys x 16 dims
  u32x4 kreg[4], vreg[4];
  auto load_k = [&](int J) {
    const uint8_t *src = kp + ((ztok + (size_t)J * kBlock + krow) * a.Hkv + w.g) * kHeadDim + 16 * kcol;
    const size_t step = (size_t)32 * a.Hkv * kHeadDim;
#pragma unroll
    for (int p = 0; p < 4; ++p) kreg[p] = ld16(src + p * step);
  };
  auto store_k = [&]() {
#pragma unroll
    for (int p = 0; p < 4; ++p) st16(&Ks[(krow + 32 * p) * kRow8 + 16 * kcol], kreg[p]);
  };
  auto load_v = [&](int J) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vreg[e] = ld16(vp + ((ztok + (size_t)J * kBlock + 4 * kg + e) * a.Hkv + w.g) * kHeadDim + 16 * dc);
  };
  auto store_v = [&]() {
    const int pos = vpos_fp8(kg);
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {   // dims 16 dc + 4 wd + (0..3)
      const uint32_t x0 = vreg[0][wd], x1 = vreg[1][wd], x2 = vreg[2][wd], x3 = vreg[3][wd];
      const uint32_t lo01 = perm_b32(x1, x0, 0x05010400u), hi01 = perm_b32(x1, x0, 0x07030602u);
      const uint32_t lo23 = perm_b32(x3, x2, 0x05010400u), hi23 = perm_b32(x3, x2, 0x07030602u);
      const int d0 = 16 * dc + 4 * wd;
      *reinterpret_cast<uint32_t *>(&Vt[(d0 + 0) * kRow8 + pos]) = perm_b32(lo23, lo01, 0x05040100u);
      *reinterpret_cast<uint32_t *>(&Vt[(d0 + 1) * kRow8 + pos]) = perm_b32(lo23, lo01, 0x07060302u);
      *reinterpret_cast<uint32_t *>(&Vt[(d0 + 2) * kRow8 + pos]) = perm_b32(hi23, hi01, 0x05040100u);
      *reinterpret_cast<uint32_t *>(&Vt[(d0 + 3) * kRow8 + pos]) = perm_b32(hi23, hi01, 0x07060302u);
    }
  };
  // The diagonal block goes to LDS as exact fp16 (every e4m3 value is an
  // fp16 value) so its P.V can use fp16 weights: the first tokens of a
  // sequence see only a handful of keys, and 3-bit weights would not average
  // out there.
  auto store_vh = [&]() {
    const int pos = vpos_bf16(kg);
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      float f[4][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const auto a01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vreg[e][wd], false);
        const auto a23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)vreg[e][wd], true);
        f[e][0] = a01[0]; f[e][1] = a01[1]; f[e][2] = a23[0]; f[e][3] = a23[1];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st8(&Vh[(16 * dc + 4 * wd + i) * kRowB + pos],
            u32x2{pack_f16x2(f[0][i], f[1][i]), pack_f16x2(f[2][i], f[3][i])});
    }
  };

  float m_run = -INFINITY, l_run = 0.f, vs_run = 1.f;
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};

  auto clampJ = [&](int x) { return x < 0 ? 0 : (x > w.I ? w.I : x); };
  int J = kSparse ? clampJ(list[0]) : 0;
  load_k(J);
  load_v(J);
  store_k();
  if (J == w.I) store_vh(); else store_v();
  __syncthreads();

  for (int b = 0; b < n_blk; ++b) {
    const bool more = b + 1 < n_blk;
    const int Jn = more ? (kSparse ? clampJ(list[b + 1]) : b + 1) : 0;
    if (more) load_k(Jn);
    const float c_blk = qs * a.k_scale[(size_t)(zrow + J) * a.Hkv + w.g];
    const float vs = a.v_scale[(size_t)(zrow + J) * a.Hkv + w.g];

    f32x16 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x16{};
      const uint8_t *kr = &Ks[(32 * tt + l32) * kRow8 + 32 * lg];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4 lo = ld16(kr + 64 * ks), hi = ld16(kr + 64 * ks + 16);
        const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s[tt] = mfma_fp8_32x32x64(av, qf[ks], s[tt]);
      }
    }

    const bool diag = (J == w.I);
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[tt][i] * c_blk;
        if (diag) {
          const int key = 32 * tt + 8 * (i >> 2) + 4 * lg + (i & 3);
          if (key > qloc) x = -INFINITY;
        }
        s[tt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = wave_max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[tt][i] - m_new);
        s[tt][i] = p * 256.f;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    const float f = alpha * (vs_run / vs);
    vs_run = vs;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[u][i] *= f;

    if (!diag) {
      i32x8 pk[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16 &st = s[2 * c + aa];
            pk[c][4 * aa + j] = (int)pack_fp8x4(st[4 * j + 0], st[4 * j + 1], st[4 * j + 2], st[4 * j + 3]);
          }
      }
      if (more) load_v(Jn);
      __syncthreads();
      if (more) store_k();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint8_t *vr = &Vt[(32 * u + l32) * kRow8 + 32 * lg];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 lo = ld16(vr + 64 * c), hi = ld16(vr + 64 * c + 16);
          const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          o[u] = mfma_fp8_32x32x64(av, pk[c], o[u]);
        }
      }
    } else {
      f16x8 pk[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int tt = c >> 1, j0 = 2 * (c & 1);
        u32x4 v4;
        v4[0] = pack_f16x2(s[tt][4 * j0 + 0], s[tt][4 * j0 + 1]);
        v4[1] = pack_f16x2(s[tt][4 * j0 + 2], s[tt][4 * j0 + 3]);
        v4[2] = pack_f16x2(s[tt][4 * j0 + 4], s[tt][4 * j0 + 5]);
        v4[3] = pack_f16x2(s[tt][4 * j0 + 6], s[tt][4 * j0 + 7]);
        pk[c] = as_f16x8(v4);
      }
      if (more) load_v(Jn);
      __syncthreads();
      if (more) store_k();
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint16_t *vr = &Vh[(32 * u + l32) * kRowB + 8 * lg];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[u] = mfma_f16_32x32x16(as_f16x8(ld16(vr + 16 * c)), pk[c], o[u]);
      }
    }
    __syncthreads();
    if (more) {
      if (Jn == w.I) store_vh(); else store_v();
    }
    J = Jn;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = vs_run / (256.f * l_tot);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 v2;
      v2[0] = pack_bf16x2(o[u][4 * jj + 0] * inv, o[u][4 * jj + 1] * inv);
      v2[1] = pack_bf16x2(o[u][4 * jj + 2] * inv, o[u][4 * jj + 3] * inv);
      st8(orow + 32 * u + 8 * jj + 4 * lg, v2);
    }
  if (a.lse && lg == 0)
    a.lse[(size_t)w.h * a.T + qtok] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
}

hipError_t launch_attn(const AttnLaunch &a, const SeqTable &t, int rows, bool sparse, bool fp8,
                       hipStream_t s) {
  const dim3 grid(rows * a.Hq), block(256);
  if (fp8) {
    if (sparse) hipLaunchKernelGGL(attn_fp8_kernel<true>, grid, block, 0, s, a, t, rows);
    else hipLaunchKernelGGL(attn_fp8_kernel<false>, grid, block, 0, s, a, t, rows);
  } else {
    if (sparse) hipLaunchKernelGGL(attn_bf16_kernel<true>, grid, block, 0, s, a, t, rows);
    else hipLaunchKernelGGL(attn_bf16_kernel<false>, grid, block, 0, s, a, t, rows);
  }
  return hipGetLastError();
}

}  // namespace stem
