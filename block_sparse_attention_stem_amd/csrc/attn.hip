// Stage 3 - causal block-sparse flash attention on gfx950 (and the dense
// baseline, which is the same tile loop over every causal block).
//
// AngelSlim doc "Stem: Rethinking Causal Information Flow in Sparse
// Attention" §2.3: exact attention on the top-k blocks only (bf16 dense and
// fp8 block-sparse prefill, varlen); youleyou HPC-BSA article §三.3.1: a
// skipped block is equivalent to -inf scores, so online softmax over just the
// listed blocks is exact.
//
// Design (per workgroup of 4 waves = one (query head h, query block I), 32
// queries per wave):
//  * Everything is computed transposed so a query lives on a lane:
//    S^T = K Q^T (A = K rows from LDS, B = the wave's Q in registers), then
//    O^T += V^T P^T (A = V^T rows from LDS, B = P^T packed straight from the
//    S^T accumulators).  With the 32x32 MFMA output layout lane l owns query
//    l % 32 in every accumulator: the row max is one cross-half exchange and
//    the O rescale is a per-lane scalar.
//  * K and V tiles reach LDS through asynchronous direct loads
//    (global_load_lds_dwordx4): no staging registers, no staging VALU.  Rows
//    are XOR-swizzled in 16-byte chunks (chunk c of row r at c ^ (r & 7)) so
//    the MFMA operand reads of 8 consecutive rows hit 8 different bank groups.
//  * V^T cannot be produced by a plain copy, so a pre-pass writes each V block
//    once per call as the exact LDS image: transposed, keys permuted into the
//    order the S^T accumulators hold them, swizzled, and (bf16 path) converted
//    to fp16, which is exact for bf16 values in fp16's range.  P.V then uses
//    fp16 weights (11 significant bits instead of bf16's 8).
//  * The next listed block's K is requested right after the current block's
//    K reads end and its V right after the V reads end, so every load has a
//    whole compute phase to land; the list is read one entry ahead and the
//    inner loop never tests whether a block is kept.
#include "stem_internal.h"
#include "gfx950_util.h"

namespace stem {

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ lds_void *lds_ptr(void *p) { return (lds_void *)p; }

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt[3:0] | expcnt 7 | lgkmcnt 15 | vmcnt[5:4]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the attention pipeline.  __syncthreads() carries a
// release fence, which on gfx9 waits for every outstanding vector-memory op,
// including the asynchronous K/V loads meant to overlap the next phase.
// Here each wave waits for its own LDS reads (lgkmcnt(0)); completion of the
// direct loads is awaited explicitly with wait_vmcnt before the barrier that
// publishes them.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void block_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);            // lgkmcnt(0), vmcnt/expcnt untouched
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Scalar (constant-address-space) view of a read-only int array: uniform
// reads become s_load, counted by lgkmcnt rather than vmcnt.
typedef const __attribute__((address_space(4))) int32_t cint32;
__device__ __forceinline__ cint32 *as_const(const int32_t *p) { return (cint32 *)p; }

constexpr int kTile16 = kBlock * kHeadDim;        // 16-bit elements in a 128x128 tile (32 KB)
constexpr int kTile8 = kBlock * kHeadDim;         // bytes in a 128x128 fp8 tile (16 KB)

// Key order inside a 16-bit V^T row: lane group x of PV step c reads the
// 8 contiguous elements 16c + 8x + 4j + r (j, r < 4), which must hold keys
// 16c + 8j + 4x + r (the S^T accumulator order).  Position -> key:
__device__ __forceinline__ int key_of_pos16(int pos) {
  const int pg = (pos >> 2) & 3;
  const int q = (pg >> 1) | ((pg & 1) << 1);
  return 16 * (pos >> 4) + 4 * q + (pos & 3);
}
// Same for an fp8 V^T row: lane group x of PV step c reads bytes
// 64c + 32x + 16a + 4j + r holding keys 64c + 32a + 8j + 4x + r.
__device__ __forceinline__ int key_of_pos8(int pos) {
  const int pg = (pos >> 2) & 15;
  const int q = (pg >> 3) | ((pg & 3) << 1) | (((pg >> 2) & 1) << 3);
  return 64 * (pos >> 6) + 4 * q + (pos & 3);
}

// ================================================================ pre-pass
// One workgroup per (global key block, KV head): V block -> LDS -> V^T image.
__global__ __launch_bounds__(256) void vprep_bf16_kernel(const __bf16 *__restrict__ v,
                                                         uint16_t *__restrict__ img, int Hkv, int R) {
  constexpr int RS = kHeadDim + 8;
  __shared__ __attribute__((aligned(16))) uint16_t tile[kBlock * RS];
  const int kb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int key = (tid >> 4) + 16 * p, ch = tid & 15;
    const u32x4 x = ld16(v + (((size_t)kb * kBlock + key) * Hkv + g) * kHeadDim + 8 * ch);
    const u32x4 y = {bf16x2_to_f16x2(x[0]), bf16x2_to_f16x2(x[1]), bf16x2_to_f16x2(x[2]),
                     bf16x2_to_f16x2(x[3])};
    st16(&tile[key * RS + 8 * ch], y);
  }
  __syncthreads();
  uint16_t *out = img + ((size_t)g * R + kb) * kTile16;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int d = (tid >> 4) + 16 * p, pch = tid & 15, lch = pch ^ (d & 7);
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[key_of_pos16(8 * lch + 2 * e) * RS + d];
      const uint32_t hi = tile[key_of_pos16(8 * lch + 2 * e + 1) * RS + d];
      w4[e] = lo | (hi << 16);
    }
    st16(out + d * kHeadDim + 8 * pch, u32x4{w4[0], w4[1], w4[2], w4[3]});
  }
}

// fp8: writes the e4m3 V^T image (16 KB per block) and an fp16 V^T image
// (32 KB per block, exact) used when the block is a row's diagonal block.
__global__ __launch_bounds__(256) void vprep_fp8_kernel(const uint8_t *__restrict__ v,
                                                        uint8_t *__restrict__ img8,
                                                        uint16_t *__restrict__ img16, int Hkv, int R) {
  constexpr int RS = kHeadDim + 16;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kBlock * RS];
  const int kb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int key = (tid >> 3) + 32 * p, ch = tid & 7;
    st16(&tile[key * RS + 16 * ch], ld16(v + (((size_t)kb * kBlock + key) * Hkv + g) * kHeadDim + 16 * ch));
  }
  __syncthreads();
  uint8_t *o8 = img8 + ((size_t)g * R + kb) * kTile8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int d = (tid >> 3) + 32 * p, pch = tid & 7, lch = pch ^ (d & 7);
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) x |= (uint32_t)tile[key_of_pos8(16 * lch + 4 * e + b) * RS + d] << (8 * b);
      w4[e] = x;
    }
    st16(o8 + d * kHeadDim + 16 * pch, u32x4{w4[0], w4[1], w4[2], w4[3]});
  }
  uint16_t *o16 = img16 + ((size_t)g * R + kb) * kTile16;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int d = (tid >> 4) + 16 * p, pch = tid & 15, lch = pch ^ (d & 7);
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __builtin_amdgcn_cvt_f32_fp8((int)tile[key_of_pos16(8 * lch + 2 * e) * RS + d], 0);
      const float hi = __builtin_amdgcn_cvt_f32_fp8((int)tile[key_of_pos16(8 * lch + 2 * e + 1) * RS + d], 0);
      w4[e] = pack_f16x2(lo, hi);
    }
    st16(o16 + d * kHeadDim + 8 * pch, u32x4{w4[0], w4[1], w4[2], w4[3]});
  }
}

// ============================================================ work decode
struct AttnItem {
  int h, g, r, z, I;
};

// Rows are walked from the last (longest causal prefix) to the first; the
// G heads of a KV group share an XCD and the chip walks one KV head at a
// time (see xcd_item).
__device__ __forceinline__ AttnItem decode_attn(const AttnLaunch &a, const SeqTable &t, int rows) {
  const int G = a.Hq / a.Hkv;
  const int item = xcd_item(blockIdx.x, rows * a.Hq, G);
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

__device__ __forceinline__ void write_out(__bf16 *orow, const f32x16 (&o)[4], float inv, int lg) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 v2;
      v2[0] = pack_bf16x2(o[u][4 * jj + 0] * inv, o[u][4 * jj + 1] * inv);
      v2[1] = pack_bf16x2(o[u][4 * jj + 2] * inv, o[u][4 * jj + 3] * inv);
      st8(orow + 32 * u + 8 * jj + 4 * lg, v2);
    }
}

__device__ __forceinline__ void write_empty(__bf16 *orow, float *lse, int lg) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) st8(orow + 32 * u + 8 * jj + 4 * lg, u32x2{0u, 0u});
  if (lse && lg == 0) *lse = -INFINITY;
}

// Online-softmax step on the raw S^T accumulators (lane = one query, 64 of
// its 128 keys; the other 64 sit in lane ^ 32).  c = this block's logit
// scale times log2 e (> 0), so the block max is c * max(raw) and every weight
// is one fma + exp2.  The running max m_run is kept in scaled (log2) units.
// Leaves p = 2^(c s - m) in s and returns the rescale factor of O.
__device__ __forceinline__ float softmax_step(f32x16 (&s)[4], bool diag, int qloc, int lg, float c,
                                              float &m_run, float &l_run) {
  if (diag) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * tt + 8 * (i >> 2) + 4 * lg + (i & 3);
        if (key > qloc) s[tt][i] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[tt][i]);
  mx = wave_max_xor32(mx);
  const float m_new = fmaxf(m_run, mx * c);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  m_run = m_new;
  float psum = 0.f;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[tt][i], c, -m_new));
      s[tt][i] = p;
      psum += p;
    }
  l_run = l_run * alpha + psum;
  return alpha;
}

// ===================================================================== bf16
template <bool kSparse>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnLaunch a, SeqTable t, int rows) {
  __shared__ __attribute__((aligned(1024))) uint16_t Ks[kTile16];   // bf16 K, [key][d] swizzled
  __shared__ __attribute__((aligned(1024))) uint16_t Vs[kTile16];   // fp16 V^T image

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 5, l32 = lane & 31, sw = l32 & 7;
  const AttnItem w = decode_attn(a, t, rows);
  const uint16_t *kp = (const uint16_t *)a.k;
  const int zrow = t.row[w.z];
  const size_t ztok = (size_t)t.tok[w.z];
  const size_t qtok0 = ztok + (size_t)w.I * kBlock;
  const int qloc = wave * 32 + l32;
  const size_t qtok = qtok0 + qloc;
  cint32 *list = kSparse ? as_const(a.idx) + ((size_t)w.h * a.R + w.r) * a.k_cap : nullptr;
  // Lists are trusted to be ascending in [0, I]; counts and ids are still
  // clamped so a malformed list can never address outside the sequence.
  int n_blk = kSparse ? as_const(a.cnt)[(size_t)w.h * a.R + w.r] : w.I + 1;
  if (kSparse && n_blk > a.k_cap) n_blk = a.k_cap;
  __bf16 *orow = (__bf16 *)a.out + (qtok * a.Hq + w.h) * kHeadDim;
  float *lse = a.lse ? a.lse + (size_t)w.h * a.T + qtok : nullptr;
  if (n_blk <= 0) {
    write_empty(orow, lse, lg);
    return;
  }
  auto clampJ = [&](int x) { return x < 0 ? 0 : (x > w.I ? w.I : x); };

  // Q as the B operand: query qloc, head dims 16 ks + 8 lg .. +7
  bf16x8 qf[8];
  {
    const __bf16 *qrow = (const __bf16 *)a.q + (qtok * a.Hq + w.h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
  }

  // Direct loads: wave w moves 8 KB of each tile, 1 KB per instruction
  // (4 rows of 256 B); lane i writes LDS bytes 16 i .. 16 i + 15.  Bases are
  // wave-uniform (scalar registers); each lane adds one fixed offset.  For K,
  // row r = 32 w + 4 j + (lane >> 4) takes its 16-byte chunk (lane & 15) ^
  // (r & 7), and r & 7 = (lane >> 4) + 4 (j & 1).
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const size_t kstride = (size_t)a.Hkv * kHeadDim;
  const uint32_t koff_even = (lane >> 4) * kstride + 8 * ((lane & 15) ^ (lane >> 4));
  const uint32_t koff_odd = (lane >> 4) * kstride + 8 * ((lane & 15) ^ ((lane >> 4) + 4));
  const uint16_t *kbase = kp + ((ztok + 32 * wv) * a.Hkv + w.g) * kHeadDim;
  const uint16_t *vbase = a.vimg16 + ((size_t)w.g * a.R + zrow) * kTile16 + (8 * wv) * 512;
  auto issue_k = [&](int J) __attribute__((always_inline)) {
    const uint16_t *src = kbase + (size_t)J * kBlock * kstride;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(src + 4 * j * kstride + ((j & 1) ? koff_odd : koff_even),
                                       lds_ptr(Ks + (8 * wv + j) * 512), 16, 0, 0);
  };
  auto issue_v = [&](int J) __attribute__((always_inline)) {
    const uint16_t *src = vbase + (size_t)J * kTile16 + lane * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(src + j * 512, lds_ptr(Vs + (8 * wv + j) * 512), 16, 0, 0);
  };
  // Swizzled operand reads: row 32 t + l32 (l32 & 7 = x), logical chunk
  // 2 k + lg sits at 2 (k ^ (x >> 1)) + (lg ^ (x & 1)); k ^ (x >> 1) only
  // permutes k's two low bits, so 4 base addresses plus immediate offsets
  // cover every read.
  const int x0 = sw & 1, x21 = sw >> 1;
  const uint16_t *kad[4], *vad[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    kad[b] = &Ks[l32 * kHeadDim + 8 * (lg ^ x0) + 16 * (b ^ x21)];
    vad[b] = &Vs[l32 * kHeadDim + 8 * (lg ^ x0) + 16 * (b ^ x21)];
  }

  const float c = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};

  // One block of the pipeline.  `issue` is a constant at each call site: the
  // loop body always prefetches the next block, the peeled last block never
  // does, so the number of loads in flight is the same on every path (the
  // compiler's wait bookkeeping then keeps the precise vmcnt(8)).
  auto step = [&](int J, int Jn, bool issue) __attribute__((always_inline)) {
    wait_vmcnt<8>();                 // this wave's K of block J has landed (V may be in flight)
    block_sync();                    // ... and every wave's
    f32x16 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[tt] = mfma_bf16_32x32x16(as_bf16x8(ld16(kad[ks & 3] + 32 * kHeadDim * tt + 64 * (ks >> 2))), qf[ks],
                                   s[tt]);
    }
    const float alpha = softmax_step(s, J == w.I, qloc, lg, c, m_run, l_run);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[u][i] *= alpha;
    }
    wait_vmcnt<0>();                 // V of block J has landed
    block_sync();                    // every wave: V landed, K reads done
    if (issue) issue_k(Jn);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int tt = cc >> 1, j0 = 8 * (cc & 1);
      const u32x4 v4 = {pack_f16x2(s[tt][j0 + 0], s[tt][j0 + 1]), pack_f16x2(s[tt][j0 + 2], s[tt][j0 + 3]),
                        pack_f16x2(s[tt][j0 + 4], s[tt][j0 + 5]), pack_f16x2(s[tt][j0 + 6], s[tt][j0 + 7])};
      const f16x8 pk = as_f16x8(v4);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[u] = mfma_f16_32x32x16(as_f16x8(ld16(vad[cc & 3] + 32 * kHeadDim * u + 64 * (cc >> 2))), pk, o[u]);
    }
    block_sync();                    // every wave is done reading V
    if (issue) issue_v(Jn);
  };

  int J = kSparse ? clampJ(list[0]) : 0;
  issue_k(J);
  issue_v(J);
  for (int b = 0; b + 1 < n_blk; ++b) {
    const int Jn = kSparse ? clampJ(list[b + 1]) : b + 1;
    step(J, Jn, true);
    J = Jn;
  }
  step(J, 0, false);

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  write_out(orow, o, 1.f / l_tot, lg);
  if (lse && lg == 0) *lse = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
}

// ====================================================================== fp8
// Same pipeline on e4m3 operands with the 32x32x64 fp8 MFMA: Q.K^T in two
// K=64 steps per key tile, P quantised to e4m3 as p * 2^8 (p <= 1, so the
// largest code is 256 < 448 and fewer small weights flush to zero), P.V in
// two K=64 steps per head-dim tile.  Per-block scales: the q and k scales
// fold into the exponent scale c of the block; the v scale of block J is
// applied by keeping O in units of the current block's v scale (one multiply
// merged with the online-softmax rescale).  The diagonal block, where the
// first queries of a sequence see only a few keys and 3-bit weights would not
// average out, runs its P.V in fp16 from the exact fp16 V^T image.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}


template <bool kSparse>
__global__ __launch_bounds__(256, 2) void attn_fp8_kernel(AttnLaunch a, SeqTable t, int rows) {
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[kTile8];      // e4m3 K, [key][d] swizzled
  __shared__ __attribute__((aligned(1024))) uint8_t Vs[kTile8];      // e4m3 V^T image
  __shared__ __attribute__((aligned(1024))) uint16_t Vh[kTile16];    // fp16 V^T image (diagonal)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 5, l32 = lane & 31, sw = l32 & 7;
  const AttnItem w = decode_attn(a, t, rows);
  const uint8_t *kp = (const uint8_t *)a.k;
  const int zrow = t.row[w.z];
  const size_t ztok = (size_t)t.tok[w.z];
  const size_t qtok0 = ztok + (size_t)w.I * kBlock;
  const int qloc = wave * 32 + l32;
  const size_t qtok = qtok0 + qloc;
  cint32 *list = kSparse ? as_const(a.idx) + ((size_t)w.h * a.R + w.r) * a.k_cap : nullptr;
  int n_blk = kSparse ? as_const(a.cnt)[(size_t)w.h * a.R + w.r] : w.I + 1;
  if (kSparse && n_blk > a.k_cap) n_blk = a.k_cap;
  __bf16 *orow = (__bf16 *)a.out + (qtok * a.Hq + w.h) * kHeadDim;
  float *lse = a.lse ? a.lse + (size_t)w.h * a.T + qtok : nullptr;
  if (n_blk <= 0) {
    write_empty(orow, lse, lg);
    return;
  }
  auto clampJ = [&](int x) { return x < 0 ? 0 : (x > w.I ? w.I : x); };

  i32x8 qf[2];
  {
    const uint8_t *qrow = (const uint8_t *)a.q + (qtok * a.Hq + w.h) * kHeadDim + 32 * lg;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 lo = ld16(qrow + 64 * ks), hi = ld16(qrow + 64 * ks + 16);
      qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }
  const float cq = a.q_scale[(size_t)w.r * a.Hq + w.h] * a.scale_log2;

  // Direct loads as in the bf16 kernel.  K rows are 128 B: row r = 32 w +
  // 8 j + (lane >> 3) takes chunk (lane & 7) ^ (r & 7) with r & 7 = lane >> 3.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const size_t kstride = (size_t)a.Hkv * kHeadDim;
  const uint32_t koff = (lane >> 3) * kstride + 16 * ((lane & 7) ^ (lane >> 3));
  const uint8_t *kbase = kp + ((ztok + 32 * wv) * a.Hkv + w.g) * kHeadDim;
  const uint8_t *v8base = a.vimg8 + ((size_t)w.g * a.R + zrow) * kTile8 + (4 * wv) * 1024;
  const uint16_t *v16base = a.vimg16 + ((size_t)w.g * a.R + zrow) * kTile16 + (8 * wv) * 512;
  auto issue_k = [&](int J) __attribute__((always_inline)) {
    const uint8_t *src = kbase + (size_t)J * kBlock * kstride + koff;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(src + 8 * j * kstride, lds_ptr(Ks + (4 * wv + j) * 1024), 16, 0, 0);
  };
  auto issue_v8 = [&](int J) __attribute__((always_inline)) {
    const uint8_t *src = v8base + (size_t)J * kTile8 + lane * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(src + j * 1024, lds_ptr(Vs + (4 * wv + j) * 1024), 16, 0, 0);
  };
  auto issue_v16 = [&](int J) __attribute__((always_inline)) {
    const uint16_t *src = v16base + (size_t)J * kTile16 + lane * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(src + j * 512, lds_ptr(Vh + (8 * wv + j) * 512), 16, 0, 0);
  };
  // Swizzled reads of 128-byte rows: logical chunk 4 k + 2 lg + e sits at
  // 4 (k ^ x2) + 2 (lg ^ x1) + (e ^ x0) for x = l32 & 7.
  const int x0 = sw & 1, x1 = (sw >> 1) & 1, x2 = sw >> 2;
  const uint8_t *k8ad[2][2], *v8ad[2][2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = 4 * (k ^ x2) + 2 * (lg ^ x1) + (e ^ x0);
      k8ad[k][e] = &Ks[l32 * kHeadDim + 16 * ch];
      v8ad[k][e] = &Vs[l32 * kHeadDim + 16 * ch];
    }
  const uint16_t *vhad[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) vhad[b] = &Vh[l32 * kHeadDim + 8 * (lg ^ x0) + 16 * (b ^ (sw >> 1))];
  auto ld32 = [](const uint8_t *lo_p, const uint8_t *hi_p) __attribute__((always_inline)) {
    const u32x4 lo = ld16(lo_p), hi = ld16(hi_p);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  float m_run = -INFINITY, l_run = 0.f, vs_run = 1.f;
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};

  // kNext: what the step prefetches for the next block (0 nothing, 1 the e4m3
  // V^T image, 2 the fp16 one for a diagonal block); kDiagPath: whether this
  // block may be the diagonal one (only the last listed block can be).
  enum { kNone = 0, kV8 = 1, kV16 = 2 };
  auto step = [&](int J, int Jn, int kNext, bool may_diag, bool v16_pending) __attribute__((always_inline)) {
    if (v16_pending) wait_vmcnt<8>(); else wait_vmcnt<4>();
    block_sync();
    const bool diag = may_diag && (J == w.I);
    const float c = cq * a.k_scale[(size_t)(zrow + J) * a.Hkv + w.g];
    const float vs = a.v_scale[(size_t)(zrow + J) * a.Hkv + w.g];
    f32x16 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        s[tt] = mfma_fp8_32x32x64(ld32(k8ad[ks][0] + 4096 * tt, k8ad[ks][1] + 4096 * tt), qf[ks], s[tt]);
    }
    const float alpha = softmax_step(s, diag, qloc, lg, c, m_run, l_run);
    const float f = alpha * (vs_run / vs);
    vs_run = vs;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[u][i] *= f;
    wait_vmcnt<0>();
    block_sync();
    if (kNext != kNone) issue_k(Jn);
    if (!diag) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        i32x8 pk;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16 &st = s[2 * cc + aa];
            pk[4 * aa + j] = (int)pack_fp8x4(st[4 * j + 0] * 256.f, st[4 * j + 1] * 256.f,
                                             st[4 * j + 2] * 256.f, st[4 * j + 3] * 256.f);
          }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[u] = mfma_fp8_32x32x64(ld32(v8ad[cc][0] + 4096 * u, v8ad[cc][1] + 4096 * u), pk, o[u]);
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int tt = cc >> 1, j0 = 8 * (cc & 1);
        const u32x4 v4 = {pack_f16x2(s[tt][j0 + 0] * 256.f, s[tt][j0 + 1] * 256.f),
                          pack_f16x2(s[tt][j0 + 2] * 256.f, s[tt][j0 + 3] * 256.f),
                          pack_f16x2(s[tt][j0 + 4] * 256.f, s[tt][j0 + 5] * 256.f),
                          pack_f16x2(s[tt][j0 + 6] * 256.f, s[tt][j0 + 7] * 256.f)};
        const f16x8 pk = as_f16x8(v4);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[u] = mfma_f16_32x32x16(as_f16x8(ld16(vhad[cc & 3] + 32 * kHeadDim * u + 64 * (cc >> 2))), pk, o[u]);
      }
    }
    block_sync();
    if (kNext == kV8) issue_v8(Jn);
    if (kNext == kV16) issue_v16(Jn);
  };

  // Lists are ascending, so only the last block can be the diagonal one: the
  // loop body handles blocks whose successor is not last; the last two steps
  // are peeled so every prefetch count is fixed at its call site.
  int J = kSparse ? clampJ(list[0]) : 0;
  const bool first_v16 = (n_blk == 1) && (J == w.I);
  issue_k(J);
  if (first_v16) issue_v16(J); else issue_v8(J);
  for (int b = 0; b + 2 < n_blk; ++b) {
    const int Jn = kSparse ? clampJ(list[b + 1]) : b + 1;
    step(J, Jn, kV8, false, false);
    J = Jn;
  }
  if (n_blk >= 2) {
    const int Jl = kSparse ? clampJ(list[n_blk - 1]) : n_blk - 1;
    if (Jl == w.I) {
      step(J, Jl, kV16, false, false);
      J = Jl;
      step(J, 0, kNone, true, true);
    } else {
      step(J, Jl, kV8, false, false);
      J = Jl;
      step(J, 0, kNone, false, false);
    }
  } else {
    if (first_v16) step(J, 0, kNone, true, true);
    else step(J, 0, kNone, false, false);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  write_out(orow, o, vs_run / (256.f * l_tot), lg);
  if (lse && lg == 0) *lse = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
}

// ================================================================ launchers
size_t attn_workspace_bytes(int Hkv, int R, bool fp8) {
  const size_t per_block = fp8 ? (size_t)kTile8 + 2 * (size_t)kTile16 : 2 * (size_t)kTile16;
  return (size_t)Hkv * R * per_block;
}

hipError_t launch_vprep(const AttnLaunch &a, bool fp8, hipStream_t s) {
  const dim3 grid(a.R, a.Hkv);
  if (fp8)
    hipLaunchKernelGGL(vprep_fp8_kernel, grid, dim3(256), 0, s, (const uint8_t *)a.v, a.vimg8, a.vimg16,
                       a.Hkv, a.R);
  else
    hipLaunchKernelGGL(vprep_bf16_kernel, grid, dim3(256), 0, s, (const __bf16 *)a.v, a.vimg16, a.Hkv, a.R);
  return hipGetLastError();
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
