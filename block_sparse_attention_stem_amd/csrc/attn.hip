// Stage 3 - causal block-sparse flash attention on gfx950 (and the dense
// baseline, which is the same tile loop over every causal block).
//
// AngelSlim doc "Stem: Rethinking Causal Information Flow in Sparse
// Attention" §2.3: exact attention on the top-k blocks only (bf16 dense and
// fp8 block-sparse prefill, varlen); youleyou HPC-BSA article §三.3.1: a
// skipped block is equivalent to -inf scores, so online softmax over just the
// listed blocks is exact.
//
// Design shared by the kernels below (one workgroup = one (query head h,
// query block row I); each wave holds 32 queries):
//  * Everything is computed transposed so a query lives on a lane:
//    S^T = K Q^T (A = K rows from LDS, B = the wave's Q in registers), then
//    O^T += V^T P^T (A = V^T rows from LDS, B = P^T packed straight from the
//    S^T accumulators).  With the 32x32 MFMA output layout lane l owns query
//    l % 32 in every accumulator: the row max is one cross-half exchange and
//    the O rescale is a per-lane scalar.
//  * K and V tiles reach LDS through asynchronous direct loads (buffer or
//    global loads with the lds modifier): no staging registers, no staging
//    VALU.  Each 1 KB instruction fills 64 consecutive 16-byte LDS slots, and
//    each lane may fetch any global chunk, so tiles are laid out with one pad
//    chunk per row (rows of 17 chunks for 256-byte rows, 9 for 128-byte
//    rows; a pad slot re-reads a valid chunk).  Row r then starts 4 (r mod 16)
//    banks further along the 64-bank LDS, so the 16 lanes served together (16
//    consecutive rows, same column) never collide, and every operand read of
//    a lane is one base address plus immediate offsets.
//  * V^T cannot be produced by a plain copy, so a pre-pass writes each V block
//    once per call as the exact LDS image: transposed, keys permuted into the
//    order the S^T accumulators hold them, padded, and (bf16 path) converted
//    to fp16, which is exact for bf16 values in fp16's range.  P.V then uses
//    fp16 weights (11 significant bits instead of bf16's 8).
//  * Loads for the next listed block are issued while the current one
//    computes, the list is read one entry ahead, and the inner loop never
//    tests whether a block is kept.
//  * bf16: 8 waves in two groups that split each block's keys and run one
//    phase apart (MFMA phase of one wave beside the softmax of the other on
//    each SIMD), one workgroup per CU.  fp8: 4 waves over all 128 keys, two
//    workgroups per CU.
#include <type_traits>

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
// publishes them.  The signal fences keep the compiler from moving memory
// accesses across the barrier (register-only work such as MFMAs may still
// cross it).
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

// Padded tile images: 128 rows of 17 (16-bit rows) or 9 (8-bit rows) 16-byte
// chunks; the last chunk of a row is padding.
constexpr int kRow16 = 136;                        // elements per 16-bit row (272 B)
constexpr int kRow8 = 144;                         // bytes per 8-bit row
constexpr int kTile16 = kBlock * kRow16;           // 16-bit elements per tile (34 KB)
constexpr int kTile8 = kBlock * kRow8;             // bytes per fp8 tile (18 KB)
constexpr int kSlots16 = kTile16 / 8;              // 16-byte slots per 16-bit tile (2176 = 34 KB)
constexpr int kSlots8 = kTile8 / 16;               // 16-byte slots per fp8 tile (1152 = 18 KB)

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
                                                         uint16_t *__restrict__ img, int Hkv, int R,
                                                         int32_t *__restrict__ ctr, int n_ctr) {
  constexpr int RS = kHeadDim + 8;
  __shared__ __attribute__((aligned(16))) uint16_t tile[kBlock * RS];
  const int kb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  if (kb == 0 && g == 0)             // the attention kernel's work queues start empty
    for (int i = tid; i < n_ctr; i += 256) ctr[i] = 0;
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
    const int d = (tid >> 4) + 16 * p, ch = tid & 15;
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[key_of_pos16(8 * ch + 2 * e) * RS + d];
      const uint32_t hi = tile[key_of_pos16(8 * ch + 2 * e + 1) * RS + d];
      w4[e] = lo | (hi << 16);
    }
    st16(out + d * kRow16 + 8 * ch, u32x4{w4[0], w4[1], w4[2], w4[3]});
  }
  if (tid < kBlock) st16(out + tid * kRow16 + kHeadDim, u32x4{0u, 0u, 0u, 0u});   // pad chunk
}

// fp8: writes the e4m3 V^T image (16 KB per block) and, unless img16 is null,
// an fp16 V^T image (32 KB per block, exact) for the fp16-weight kernel.
// Block kb (global key-block row, the image index) starts at token tb of v.
__device__ __forceinline__ void vprep_fp8_block(const uint8_t *__restrict__ v, size_t tb, int kb, int g,
                                                uint8_t *__restrict__ img8, uint16_t *__restrict__ img16,
                                                int Hkv, int R, uint8_t *tile) {
  constexpr int RS = kHeadDim + 16;
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int key = (tid >> 3) + 32 * p, ch = tid & 7;
    st16(&tile[key * RS + 16 * ch], ld16(v + ((tb + key) * Hkv + g) * kHeadDim + 16 * ch));
  }
  __syncthreads();
  uint8_t *o8 = img8 + ((size_t)g * R + kb) * kTile8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int d = (tid >> 3) + 32 * p, ch = tid & 7;
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) x |= (uint32_t)tile[key_of_pos8(16 * ch + 4 * e + b) * RS + d] << (8 * b);
      w4[e] = x;
    }
    st16(o8 + d * kRow8 + 16 * ch, u32x4{w4[0], w4[1], w4[2], w4[3]});
  }
  if (tid < kBlock) st16(o8 + tid * kRow8 + kHeadDim, u32x4{0u, 0u, 0u, 0u});
  if (img16 == nullptr) return;
  uint16_t *o16 = img16 + ((size_t)g * R + kb) * kTile16;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int d = (tid >> 4) + 16 * p, ch = tid & 15;
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = __builtin_amdgcn_cvt_f32_fp8((int)tile[key_of_pos16(8 * ch + 2 * e) * RS + d], 0);
      const float hi = __builtin_amdgcn_cvt_f32_fp8((int)tile[key_of_pos16(8 * ch + 2 * e + 1) * RS + d], 0);
      w4[e] = pack_f16x2(lo, hi);
    }
    st16(o16 + d * kRow16 + 8 * ch, u32x4{w4[0], w4[1], w4[2], w4[3]});
  }
  if (tid < kBlock) st16(o16 + tid * kRow16 + kHeadDim, u32x4{0u, 0u, 0u, 0u});
}

__global__ __launch_bounds__(256) void vprep_fp8_kernel(const uint8_t *__restrict__ v,
                                                        uint8_t *__restrict__ img8,
                                                        uint16_t *__restrict__ img16, int Hkv, int R,
                                                        int32_t *__restrict__ ctr, int n_ctr) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kBlock * (kHeadDim + 16)];
  const int kb = blockIdx.x, g = blockIdx.y;
  if (kb == 0 && g == 0)             // the attention kernel's work queues start empty
    for (int i = threadIdx.x; i < n_ctr; i += 256) ctr[i] = 0;
  vprep_fp8_block(v, (size_t)kb * kBlock, kb, g, img8, img16, Hkv, R, tile);
}

// Paged: row kb_local of this launch's sequences reads its tokens from the
// page its sequence's table names (clamped into the pool), and copies that
// page's K and V scales to the row-indexed arrays ksr / vsr [R][Hkv], so the
// attention kernel looks scales up by row exactly as for contiguous K/V.
__global__ __launch_bounds__(256) void vprep_fp8_paged_kernel(const uint8_t *__restrict__ v,
                                                              uint8_t *__restrict__ img8,
                                                              uint16_t *__restrict__ img16, int Hkv, int R,
                                                              const int32_t *__restrict__ table,
                                                              int table_stride, int num_pages, SeqTable t,
                                                              const float *__restrict__ ksp,
                                                              const float *__restrict__ vsp,
                                                              float *__restrict__ ksr, float *__restrict__ vsr,
                                                              int32_t *__restrict__ ctr) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kBlock * (kHeadDim + 16)];
  const int kb = t.row[0] + blockIdx.x, g = blockIdx.y;
  if (blockIdx.x == 0 && g == 0 && threadIdx.x < 8) ctr[threadIdx.x] = 0;   // this launch's work queues
  const int z = seq_of(t.row, t.n, kb);
  int page = table[(size_t)(t.z0 + z) * table_stride + (kb - t.row[z])];
  page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
  if (threadIdx.x == 0) {
    ksr[(size_t)kb * Hkv + g] = ksp[(size_t)page * Hkv + g];
    vsr[(size_t)kb * Hkv + g] = vsp[(size_t)page * Hkv + g];
  }
  vprep_fp8_block(v, (size_t)page * kBlock, kb, g, img8, img16, Hkv, R, tile);
}

// ============================================================ work decode
struct AttnItem {
  int h, g, r, z, I;
};

// Items are ordered by KV group, then by row from the last (longest causal
// prefix) to the first, then by the G query heads of the group; each XCD
// takes a contiguous eighth of that order (xcd_chunk_item), so its L2 serves
// neighbouring rows of one KV group, which list mostly the same blocks.
__device__ __forceinline__ AttnItem decode_item(const AttnLaunch &a, const SeqTable &t, int rows, int item) {
  const int G = a.Hq / a.Hkv;
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

// The output tile goes out through LDS: in the MFMA layout a lane holds one
// query's dims in 8-byte pieces, and the query rows of [T][Hq][d] lie
// Hq * d * 2 bytes apart, so direct stores would touch 32 rows per
// instruction.  stage_out writes the bf16 tile [128 queries][136] (8 pad
// elements per row) into free LDS; store_staged then writes whole 256-byte
// query rows, 16 lanes per row.
constexpr int kOutRow = kHeadDim + 8;
__device__ __forceinline__ void stage_out(uint16_t *stg, const f32x16 (&o)[4], int qloc, int lg) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 v2;
      v2[0] = pack_bf16x2(o[u][4 * jj + 0], o[u][4 * jj + 1]);
      v2[1] = pack_bf16x2(o[u][4 * jj + 2], o[u][4 * jj + 3]);
      st8(stg + qloc * kOutRow + 32 * u + 8 * jj + 4 * lg, v2);
    }
}
template <int kThreads>
__device__ __forceinline__ void store_staged(const uint16_t *stg, __bf16 *out0, int Hq, int tid) {
#pragma unroll
  for (int it = 0; it < kBlock * 16 / kThreads; ++it) {
    const int c = it * kThreads + tid, row = c >> 4, ch = c & 15;
    st16(out0 + (size_t)row * Hq * kHeadDim + 8 * ch, ld16(stg + row * kOutRow + 8 * ch));
  }
}

__device__ __forceinline__ void write_empty(__bf16 *orow, float *lse, int lg) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) st8(orow + 32 * u + 8 * jj + 4 * lg, u32x2{0u, 0u});
  if (lse && lg == 0) *lse = -INFINITY;
}

// Online-softmax step of the fp8 kernel on the raw S^T accumulators (lane =
// one query, 64 of its 128 keys; the other 64 sit in lane ^ 32).  c = the
// block's logit scale times log2 e (> 0); lv = log2 of the block's V scale.
// The V scale is folded into the weights: the MFMA operand for key k is
//   P'_k = 2^(c s_k + lv - R + kFp8Off),
// so O accumulates P' times the raw V codes, and L accumulates P'_k / vs,
// i.e. 2^(c s_k - R + kFp8Off).  Then O / L is the output and
// R - kFp8Off + log2 L the log2-sum-exp.  The reference R is raised only when
// a block's largest log-weight c s + lv exceeds it by more than kFp8Lazy
// (O and L are then rescaled), so P' <= 2^(kFp8Off + kFp8Lazy) = 430 < 448
// (the e4m3 maximum) while the largest weight seen so far keeps
// P' >= 2^(kFp8Off - kFp8Lazy) = 152: small weights stay in e4m3's normal
// range as far down as with P' = 256 p.  O is rarely touched.  Leaves P' in s
// and returns cm, the query's largest logit in the block times c.
//
// A block is heavy for a query when its largest weight is more than kHeavy
// of the query's weight sum so far, this block included (heavy_block).
// An e4m3 weight carries a relative error of up to 2^-4; spread over many
// keys of similar weight these errors average out, but when a few keys hold
// a query's attention they do not, and the fp8 kernel then adds a second
// e4m3 pass with the rounding residual of the weights (see pack_lo_fp8x4).
constexpr float kFp8Lazy = 0.75f;
constexpr float kFp8Off = 8.f;
__device__ __forceinline__ float softmax_fp8(f32x16 (&s)[4], bool diag, int qloc, int lg, float c, float lv,
                                             float inv_vs, float &R, float &L, f32x16 (&o)[4]) {
  if (diag) {
    const int lim = qloc - 4 * lg;          // key > qloc  <=>  (key - 4 lg) > lim
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        s[tt][i] = (32 * tt + 8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : s[tt][i];
  }
  float mx = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[tt][i]);
  // every query sees at least one key of the block (all of an earlier block,
  // itself in the diagonal one), so cm and mz are finite.  (The two halves of
  // the query meet through an LDS lane shuffle: v_permlane32_swap needs two
  // more VALU copies, and this kernel is bound by its VALU issue.)
  const float cm = wave_max_xor32(mx) * c;
  const float mz = cm + lv;
  if (__any(mz > R + kFp8Lazy)) {
    const float Rn = fmaxf(R, mz);
    const float f = __builtin_amdgcn_exp2f(R - Rn);   // 0 on the first block (R = -inf), else <= 1
    R = Rn;
    L *= f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[u][i] *= f;
  }
  const float off = lv - R + kFp8Off;
  float psum = 0.f;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[tt][i], c, off));
      s[tt][i] = p;
      psum += p;
    }
  L = fmaf(psum, inv_vs, L);
  return cm;
}

// Whether the block is heavy for this query (see softmax_fp8): its largest
// weight 2^(cm - R + kFp8Off) (L units) is more than kHeavy of l_tot, the
// query's weight sum so far (both lane halves).
constexpr float kHeavy = 0.125f;
__device__ __forceinline__ bool heavy_block(float cm, float R, float l_tot) {
  return __builtin_amdgcn_exp2f(cm - R + kFp8Off) > kHeavy * l_tot;
}

// ===================================================================== bf16
// One workgroup of 8 waves per (query head, query block), one workgroup per
// CU.  Waves w and w + 4 share a SIMD and (square rows) the same 32 queries
// (w & 3); wave w (group 0) takes keys 0-63 of every listed block, wave w + 4
// (group 1) keys 64-127, each with its own online softmax, merged once per
// row.  A group loads only its own halves of the K and V^T tiles.
//
// Ping-pong.  A wave alternates an MFMA phase M_b = (P.V of block b-1, then
// S^T = K Q^T of block b) and a VALU phase X_b = (softmax of block b: mask,
// max, lazy O rescale, exp2, fp16 packing of P), with a barrier after each.
// Both groups run the same code, but group 1 passes one extra barrier first,
// so it stays exactly one phase behind: on every SIMD one wave's exponentials
// overlap the other wave's MFMAs.
//
// Buffers.  Block b's K half sits in K[b % 2] and its V half in V[b % 2]
// (separate LDS arrays, so the compiler sees that reads never alias loads in
// flight).  During M_b a group requests K of block b+1 and V of block b;
// both have the rest of M_b and X_b to land and are awaited before the
// barrier that opens M_{b+1}.
//
// O is rescaled lazily: the running max used for the weights is raised only
// when a block's max exceeds it by more than 2^8 (weights stay <= 256, exact
// range for fp16), which skips almost every rescale.
//
// kPair: 64 x 128 blocks (64-query rows, 128-key blocks).  A workgroup still
// runs the 128-query tile of block row r, but each 64-query half has its own
// list (list rows 2r and 2r + 1): the tile walks the ascending union of the
// two lists, built once per workgroup in LDS (a bitmap per half, then one
// wave compacts their OR in ascending order).  The waves are laid out so
// that a half can be skipped without idling a SIMD: group g holds the 64
// queries of half g (waves 4g + {0, 1}: keys 0-63, waves 4g + {2, 3}: keys
// 64-127), so every SIMD runs one wave of each half.  A wave skips the S^T
// MFMAs and the softmax of a block its half does not own, and the P.V MFMAs
// of that block one phase later; only its loads still go.  Group 0 issues
// the loads of both key halves (group 1 reads a tile one phase after group 0
// has waited for it), and the two groups keep the square-row ping-pong.
// Measured on the 128K layer (~25 % of pairs per half): identical half lists
// cost 1.10x the square-row call per computed pair, independent half lists
// (union ~39 % of the blocks) 1.37x per computed pair; without the skip the
// time follows the union (1.59x per pair).  A half-owned block still takes
// two phases, in which the owning wave's MFMAs and softmax no longer overlap
// with the other wave's, which is the remaining cost.
constexpr float kLazyLog2 = 8.f;
constexpr int kHalfK = 64 * kRow16;              // K half: 64 keys x 17 chunks (elements)
constexpr int kRowVh = 72;                       // V^T half row: 64 keys + pad chunk (elements)
constexpr int kHalfV = kHeadDim * kRowVh;        // V^T half: 128 dims x 9 chunks (elements)
constexpr uint32_t kBufWord3 = 0x00020000u;      // raw buffer descriptor word 3 (gfx9 dword access)

template <bool kSparse, bool kPair, typename Claim>
__device__ __forceinline__ void attn_bf16_item(const AttnLaunch &a, const SeqTable &t, int rows, int item,
                                               Claim &&claim) {
  static_assert(kSparse || !kPair, "paired lists are block-sparse");
  __shared__ __attribute__((aligned(1024))) uint16_t K0[2 * kHalfK];   // bf16 K halves, [key][d]
  __shared__ __attribute__((aligned(1024))) uint16_t V0[2 * kHalfV];   // fp16 V^T halves, [d][key]
  __shared__ __attribute__((aligned(1024))) uint16_t K1[2 * kHalfK];
  __shared__ __attribute__((aligned(1024))) uint16_t V1[2 * kHalfV];
  // kPair: union list (block | ownership << 16) and the two ownership bitmaps
  __shared__ int32_t Ulist[kPair ? kMaxListBlocks : 1];
  __shared__ uint32_t Ubits[kPair ? 2 * (kMaxListBlocks / 32) + 1 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int lg = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Loader roles: wave (qw, kh) issues share qw of the tile loads of key
  // half kh.  Compute roles: grp is the ping-pong group, cq the wave's
  // 32-query slice and ck its key half.  Square rows: cq = qw, ck = grp = kh.
  // kPair: group g holds the 64 queries of half g and spreads them over all
  // four SIMDs (ck = bit 1 of the wave), so a block listed for one half only
  // still gives every SIMD MFMA work.
  const int qw = wv & 3, kh = wv >> 2;
  const int grp = kh;
  const int cq = kPair ? 2 * grp + (wv & 1) : qw;
  const int ck = kPair ? ((wv >> 1) & 1) : kh;
  const AttnItem w = decode_item(a, t, rows, item);
  const int zrow = t.row[w.z];
  const size_t ztok = (size_t)t.tok[w.z];
  const size_t qtok0 = ztok + (size_t)w.I * kBlock;
  const int qloc = cq * 32 + l32;
  const size_t qtok = qtok0 + qloc;
  // kPair: list rows 2r (queries 0-63) and 2r + 1 (queries 64-127)
  const size_t lrow = kPair ? ((size_t)w.h * a.R + w.r) * 2 : (size_t)w.h * a.R + w.r;
  cint32 *list = kSparse ? as_const(a.idx) + lrow * a.k_cap : nullptr;
  // Lists are trusted to be ascending in [0, I]; counts and ids are still
  // clamped so a malformed list can never address outside the sequence.
  // The first entry is read beside the count (a list row always has k_cap
  // entries, so it exists even when the count is 0) and Q is requested
  // before either arrives: a row then starts after one scalar round trip
  // and one tile fetch, not three dependent fetches.
  int n_blk = kSparse ? as_const(a.cnt)[lrow] : w.I + 1;
  const int first_entry = kSparse && !kPair ? list[0] : 0;
  bf16x8 qf[8];            // Q as the B operand: query qloc, head dims 16 ks + 8 lg .. +7
  {
    const __bf16 *qrow = (const __bf16 *)a.q + (qtok * a.Hq + w.h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
  }
  if (kSparse && n_blk > a.k_cap) n_blk = a.k_cap;
  int n_b = 0;
  if constexpr (kPair) {
    n_b = as_const(a.cnt)[lrow + 1];
    if (n_b > a.k_cap) n_b = a.k_cap;
    if (n_blk < 0) n_blk = 0;
    if (n_b < 0) n_b = 0;
  }
  __bf16 *orow = (__bf16 *)a.out + (qtok * a.Hq + w.h) * kHeadDim;
  float *lse = a.lse ? a.lse + (size_t)w.h * a.T + qtok : nullptr;
  if (n_blk + n_b <= 0) {
    if (ck == 0) write_empty(orow, lse, lg);
    block_sync();
    claim();
    block_sync();
    return;
  }
  auto clampJ = [&](int J) { return J < 0 ? 0 : (J > w.I ? w.I : J); };
  if constexpr (kPair) {
    // Union of the two lists: set the ownership bits of every listed block
    // (ids clamped into [0, I]), then wave 0 writes the set blocks in
    // ascending order with their ownership (bit 0: list 2r, bit 1: 2r + 1).
    const int nwords = (w.I + 1 + 31) >> 5;            // I < kMaxListBlocks (checked on the host)
    for (int i = tid; i < 2 * nwords; i += 512) Ubits[i] = 0u;
    __syncthreads();
    cint32 *list_b = list + a.k_cap;
    for (int i = tid; i < n_blk; i += 512) {
      const int J = clampJ(list[i]);
      atomicOr(&Ubits[J >> 5], 1u << (J & 31));
    }
    for (int i = tid; i < n_b; i += 512) {
      const int J = clampJ(list_b[i]);
      atomicOr(&Ubits[nwords + (J >> 5)], 1u << (J & 31));
    }
    __syncthreads();
    if (tid < 64) {
      int base = 0;
      for (int c = 0; c < nwords; c += 64) {
        const int wi = c + lane;
        const uint32_t b0 = wi < nwords ? Ubits[wi] : 0u, b1 = wi < nwords ? Ubits[nwords + wi] : 0u;
        uint32_t bits = b0 | b1;
        const int n = __popc(bits);
        int incl = n;                                  // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int y = __shfl_up(incl, d, 64);
          if (lane >= d) incl += y;
        }
        int pos = base + incl - n;
        while (bits) {
          const int bb = __ffs(bits) - 1;
          bits &= bits - 1;
          Ulist[pos++] = (32 * wi + bb) | (int)(((b0 >> bb) & 1u) | (((b1 >> bb) & 1u) << 1)) << 16;
        }
        base += __shfl(incl, 63, 64);
      }
      if (lane == 0) Ubits[2 * (kMaxListBlocks / 32)] = (uint32_t)base;
    }
    __syncthreads();
    n_blk = __builtin_amdgcn_readfirstlane((int)Ubits[2 * (kMaxListBlocks / 32)]);
  }
  // Block id b of the walk (kPair: its union entry, ownership in bits 16-17).
  auto blk_entry = [&](int b) __attribute__((always_inline)) {
    if constexpr (kPair) return __builtin_amdgcn_readfirstlane(Ulist[b]);
    else return kSparse ? clampJ(list[b]) : b;
  };
  auto blk = [&](int b) __attribute__((always_inline)) { return blk_entry(b) & 0xffff; };
  const int my_bit = grp == 0 ? 1 : 2;

  // Direct loads through raw buffer descriptors rebased per block (32-bit
  // per-lane offsets, scalar bases).  Load instruction k of a half writes
  // LDS slots 64 k + lane (16 B each); group wave qw issues k = qw + 4 m.
  //   K half: 17 loads; slot s -> key row s / 17, chunk s % 17 (chunk 16 is
  //           the pad and re-reads chunk 0).
  //   V half: 18 loads; slot s -> dim row s / 9, chunk s % 9 of this half's
  //           8 image chunks (chunk 8 is the pad and re-reads chunk 0).
  // kPair: group 0 issues the loads of both key halves and group 1 none.
  // Group 0 waits for its loads before the barrier that opens its MFMA phase
  // of the block, and group 1 reads the tile one phase later, so every wave
  // that reads a half (both groups read both) finds it landed.
  constexpr int kLdH = kPair ? 2 : 1;              // key halves a loading wave issues
  const bool loader = !kPair || grp == 0;
  const uint32_t kstride_b = (uint32_t)a.Hkv * kHeadDim * 2;
  const int nkk = qw == 0 ? 5 : 4, nkv = qw < 2 ? 5 : 4;
  const int ldh = kPair ? 0 : kh;                  // first key half this wave loads
  uint32_t koff[5], voff[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int sk = 64 * (qw + 4 * m) + lane;
    const int rk = sk / 17, chk = sk - 17 * rk;
    koff[m] = (uint32_t)rk * kstride_b + 16 * (chk < 16 ? chk : 0);
    const int sv = 64 * (qw + 4 * m) + lane;
    const int rv = sv / 9, cv = sv - 9 * rv;
    voff[m] = (uint32_t)(rv * kRow16 * 2 + 16 * (8 * ldh + (cv < 8 ? cv : 0)));
  }
  const char *kbase = (const char *)a.k + ((ztok + 64 * ldh) * a.Hkv + w.g) * kHeadDim * 2;
  const char *vbase = (const char *)(a.vimg16 + ((size_t)w.g * a.R + zrow) * kTile16);
  // K of block J, key half ldh + hh (a descriptor of size 0 when !has:
  // no memory is read and the buffer gets zeros).  Block ids are
  // wave-uniform; readfirstlane keeps the descriptors in SGPRs.
  auto k_rsrc = [&](int J, bool has, int hh) __attribute__((always_inline)) {
    J = __builtin_amdgcn_readfirstlane(J);
    return __builtin_amdgcn_make_buffer_rsrc(
        (void *)(kbase + ((size_t)J * kBlock + 64 * hh) * kstride_b), (short)0, has ? (int)(64 * kstride_b) : 0,
        kBufWord3);
  };
  auto issue_k = [&](int J, uint16_t *Kd) __attribute__((always_inline)) {
    if (!loader) return;
#pragma unroll
    for (int hh = 0; hh < kLdH; ++hh) {
      const __amdgpu_buffer_rsrc_t r = k_rsrc(J, true, hh);
      uint16_t *d = Kd + (ldh + hh) * kHalfK;
#pragma unroll
      for (int m = 0; m < 5; ++m)
        if (m < nkk) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(d + (qw + 4 * m) * 512), 16, koff[m], 0, 0, 0);
    }
  };
  auto v_rsrc = [&](int J, int hh) __attribute__((always_inline)) {
    J = __builtin_amdgcn_readfirstlane(J);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + (size_t)J * kTile16 * 2 + 128 * hh), (short)0,
                                             kTile16 * 2 - 128 * hh, kBufWord3);
  };

  const float c = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};
  f32x16 s[2];            // S^T of the current block (this wave's 64 keys)
  u32x4 pk[4];            // P of the previous block, fp16, one 16-key step each

  // MFMA phase: P.V of the previous block (if kPV) from the V^T half in Vp,
  // then S^T of this block from the K half in Kc, as one stream of MFMAs
  // whose LDS operand reads run kAhead MFMAs ahead (LDS latency under load
  // is several MFMA durations).  Consecutive MFMAs use independent
  // accumulators: P.V steps go (16-key step cc, dim tile u) with u inner,
  // S^T steps go (head-dim step ks, key tile tt) with tt inner.  The step's
  // ten direct loads are spread through the stream (one every third MFMA):
  // issued back to back they stall the wave on the memory issue queue.  The
  // wave raises its priority for the phase, so that on its SIMD its MFMAs and
  // operand reads issue ahead of the other wave's softmax VALU work (measured
  // 4 % on the 128K layer).
  constexpr int kAhead = 8;
  // kPair: a wave skips the P.V MFMAs of a block its half does not own
  // (kPV false) and the S^T MFMAs likewise (kQK false); its loads still go.
  // The loads of one block step, d = 0 .. 10 kLdH - 1: K loads of the next
  // block's halves (five per half), then V loads of this block's halves.
  auto mfma_phase = [&](auto kPV, const uint16_t *Vp, const uint16_t *Kc, int J, int Jn, bool has_next,
                        uint16_t *Kn, uint16_t *Vc, bool pv_on, bool qk_on)
                        __attribute__((always_inline)) {
    constexpr bool PV = decltype(kPV)::value;
    const __amdgpu_buffer_rsrc_t rk0 = k_rsrc(Jn, has_next, 0);
    const __amdgpu_buffer_rsrc_t rk1 = k_rsrc(Jn, has_next, kLdH - 1);
    // kPair: V half 1 through a descriptor 8 chunks on (an instruction offset
    // would move the LDS destination as well)
    const __amdgpu_buffer_rsrc_t rv = v_rsrc(J, 0);
    const __amdgpu_buffer_rsrc_t rv1 = v_rsrc(J, kLdH - 1);
    auto dma = [&](int d) __attribute__((always_inline)) {
      if (!loader) return;
      if (d < 5 * kLdH) {
        const int hh = d / 5, m = d % 5;
        if (m < nkk)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(hh ? rk1 : rk0, lds_ptr(Kn + (ldh + hh) * kHalfK + (qw + 4 * m) * 512),
                                                   16, koff[m], 0, 0, 0);
      } else {
        const int e = d - 5 * kLdH, hh = e / 5, m = e % 5;
        if (m < nkv)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(hh ? rv1 : rv, lds_ptr(Vc + (ldh + hh) * kHalfV + (qw + 4 * m) * 512),
                                                   16, voff[m], 0, 0, 0);
      }
    };
    const uint16_t *vad = Vp + ck * kHalfV + l32 * kRowVh + 8 * lg;
    const uint16_t *kad = Kc + ck * kHalfK + l32 * kRow16 + 8 * lg;
    auto rd = [&](int i) __attribute__((always_inline)) {
      return i < 16 ? ld16(vad + 32 * kRowVh * (i & 3) + 16 * (i >> 2))
                    : ld16(kad + 32 * kRow16 * ((i - 16) & 1) + 16 * ((i - 16) >> 1));
    };
    auto mfma = [&](int i, const u32x4 &x) __attribute__((always_inline)) {
      if (i < 16) {
        o[i & 3] = mfma_f16_32x32x16(as_f16x8(x), as_f16x8(pk[i >> 2]), o[i & 3]);
      } else {
        const int tt = (i - 16) & 1, ks = (i - 16) >> 1;
        s[tt] = mfma_bf16_32x32x16(as_bf16x8(x), qf[ks], ks == 0 ? f32x16{} : s[tt]);
      }
    };
    u32x4 r[32];
    __builtin_amdgcn_s_setprio(1);
    if constexpr (!kPair) {
      constexpr int i0 = PV ? 0 : 16;
#pragma unroll
      for (int i = i0; i < i0 + kAhead; ++i) r[i] = rd(i);
#pragma unroll
      for (int i = i0; i < 32; ++i) {
        if (i + kAhead < 32) r[i + kAhead] = rd(i + kAhead);
        if (PV ? (i % 3 == 1 && i < 30) : (i - 16 < 10)) dma(PV ? i / 3 : i - 16);
        __builtin_amdgcn_sched_barrier(0);
        mfma(i, r[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Two parts, P.V (MFMAs 0-15, with the K loads d = 0..9) and S^T
      // (MFMAs 16-31, with the V loads d = 10..19), each run or skipped
      // as a whole; a skipped part still issues its loads.
      auto part = [&](auto kPart, bool on) __attribute__((always_inline)) {
        constexpr int p0 = 16 * decltype(kPart)::value, d0 = 10 * decltype(kPart)::value;
        if (on) {
#pragma unroll
          for (int i = p0; i < p0 + kAhead; ++i) r[i] = rd(i);
#pragma unroll
          for (int i = p0; i < p0 + 16; ++i) {
            if (i + kAhead < p0 + 16) r[i + kAhead] = rd(i + kAhead);
            if (i - p0 < 10) dma(d0 + i - p0);
            __builtin_amdgcn_sched_barrier(0);
            mfma(i, r[i]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int d = d0; d < d0 + 10; ++d) dma(d);
          // a skipped S^T is never read (its softmax is skipped too): an
          // unspecified value keeps the old one from staying live
          if constexpr (decltype(kPart)::value == 1) {
            s[0] = __builtin_nondeterministic_value(s[0]);
            s[1] = __builtin_nondeterministic_value(s[1]);
          }
        }
      };
      part(std::integral_constant<int, 0>{}, PV && pv_on);
      part(std::integral_constant<int, 1>{}, qk_on);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // P.V of the last block (no S^T after it).
  auto pv_last = [&](const uint16_t *Vp) __attribute__((always_inline)) {
    const uint16_t *vad = Vp + ck * kHalfV + l32 * kRowVh + 8 * lg;
    u32x4 r[16];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) r[i] = ld16(vad + 32 * kRowVh * (i & 3) + 16 * (i >> 2));
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + kAhead < 16) r[i + kAhead] = ld16(vad + 32 * kRowVh * ((i + kAhead) & 3) + 16 * ((i + kAhead) >> 2));
      __builtin_amdgcn_sched_barrier(0);
      o[i & 3] = mfma_f16_32x32x16(as_f16x8(r[i]), as_f16x8(pk[i >> 2]), o[i & 3]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax of the block whose S^T is in s (lane: 32 of the query's 64 keys
  // in this half).  A query can see no key at all in this half (diagonal
  // block, keys 64-127, queries < 64): its max stays -inf, alpha stays 1 and
  // the exponent offset is 0, so every weight is 0.
  auto softmax = [&](bool diag, bool off) __attribute__((always_inline)) {
    if (off) {                     // kPair: not in this half's list (its P.V is skipped too)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) pk[cc] = __builtin_nondeterministic_value(pk[cc]);
      return;
    }
    if (diag) {
      const int lim = qloc - 64 * ck - 4 * lg;        // key > qloc  <=>  local key offset > lim
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[tt][i] = (32 * tt + 8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : s[tt][i];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[tt][i]);
    mx = wave_max_xor32(mx) * c;
    if (__any(mx > m_run + kLazyLog2)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[u][i] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[tt][i] = __builtin_amdgcn_exp2f(fmaf(s[tt][i], c, -m_use));
        psum += s[tt][i];
      }
    l_run += psum;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int tt = cc >> 1, j0 = 8 * (cc & 1);
      pk[cc] = u32x4{pack_f16x2(s[tt][j0 + 0], s[tt][j0 + 1]), pack_f16x2(s[tt][j0 + 2], s[tt][j0 + 3]),
                     pack_f16x2(s[tt][j0 + 4], s[tt][j0 + 5]), pack_f16x2(s[tt][j0 + 6], s[tt][j0 + 7])};
    }
  };

  // Block b: [wait, barrier, loads for b+1, M_b, barrier, X_b].  Block b
  // uses K[b % 2] and V[b % 2]; P.V of block b-1 reads V[(b-1) % 2].
  // kPair: ownership (bits 16-17) of the current block and of the previous one
  int own = 0, own_prev = 0;
  using NoPV = std::integral_constant<bool, false>;
  using WithPV = std::integral_constant<bool, true>;
  auto step = [&](auto kPV, int b, int &J, const uint16_t *Kc, const uint16_t *Vp, uint16_t *Kn, uint16_t *Vc)
                  __attribute__((always_inline)) {
    const int en = b + 1 < n_blk ? blk_entry(b + 1) : 0;
    const int Jn = kPair ? (en & 0xffff) : en;
    wait_vmcnt<0>();                 // this wave's K of b and V of b-1 have landed
    block_sync();                    // ... the whole group's too; Kn and Vc are free
    const bool has_next = b + 1 < n_blk;
    const bool qk_on = !kPair || ((own >> 16) & my_bit);
    const bool pv_on = !kPair || ((own_prev >> 16) & my_bit);
    mfma_phase(kPV, Vp, Kc, J, Jn, has_next, Kn, Vc, pv_on, qk_on);
    block_sync();
    softmax(J == w.I, !qk_on);
    J = Jn;
    own_prev = own;
    own = en;
  };

  if constexpr (kPair) own = blk_entry(0);
  int J = kPair ? blk(0) : (kSparse ? clampJ(first_entry) : 0);
  issue_k(J, K0);
  if (grp == 1) block_sync();        // group 1 runs one phase behind
  step(NoPV{}, 0, J, K0, V1, K1, V0);
  claim();
  int b = 1;
  while (b < n_blk) {
    step(WithPV{}, b, J, K1, V0, K0, V1);
    if (++b == n_blk) break;
    step(WithPV{}, b, J, K0, V1, K1, V0);
    ++b;
  }
  // P.V of the last block, from V[(n_blk - 1) % 2]; every load has landed
  wait_vmcnt<0>();
  block_sync();
  if (!kPair || ((own_prev >> 16) & my_bit)) pv_last((n_blk & 1) ? V0 : V1);
  if (grp == 0) block_sync();        // realign the groups

  // merge the two key halves: the key-half-1 wave of each query slice (ck = 1)
  // hands (O, m, l) to its key-half-0 partner through LDS.  Each lane's 66
  // values form one row of 68 floats (272 bytes, so the 16 lanes of a 16-byte
  // access hit distinct banks), written and read in 16-byte pieces; the
  // reader issues all of its reads before it uses any, so their latencies
  // overlap (one register reused for every read had them run one by one).
  block_sync();
  constexpr int kXRow = 68;
  float *xrow = (float *)(cq < 2 ? K0 : K1) + (cq & 1) * (64 * kXRow) + lane * kXRow;
  if (ck == 1) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        st16(xrow + 16 * u + 4 * j, u32x4{__float_as_uint(o[u][4 * j]), __float_as_uint(o[u][4 * j + 1]),
                                          __float_as_uint(o[u][4 * j + 2]), __float_as_uint(o[u][4 * j + 3])});
    st8(xrow + 64, u32x2{__float_as_uint(m_run), __float_as_uint(l_run)});
  }
  block_sync();
  if (ck == 0) {
    u32x4 xo[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) xo[k] = ld16(xrow + 4 * k);
    const u32x2 ml = *reinterpret_cast<const u32x2 *>(xrow + 64);
    // the merged max is finite: the key equal to the query is visible in one half
    const float m1 = __uint_as_float(ml[0]), l1 = __uint_as_float(ml[1]);
    const float m = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
    float l = l_run * a0 + l1 * a1;
    l += __shfl_xor(l, 32, 64);
    // kPair: a half whose list is empty sees no key (l = 0): output 0, lse -inf
    const float inv = kPair ? (l > 0.f ? 1.f / l : 0.f) : 1.f / l;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[u][i] = (o[u][i] * a0 + __uint_as_float(xo[4 * u + (i >> 2)][i & 3]) * a1) * inv;
    stage_out(V0, o, qloc, lg);
    if (lse && lg == 0) *lse = kPair && !(l > 0.f) ? -INFINITY : (m + __log2f(l)) * 0.69314718055994531f;
  }
  block_sync();
  store_staged<512>(V0, (__bf16 *)a.out + (qtok0 * a.Hq + w.h) * kHeadDim, a.Hq, tid);
}

// The bf16 kernel is persistent: one workgroup per CU (its LDS admits no
// second one) loops over (head, query block) items.  Items are ordered KV
// group, then row (longest causal prefix first), then the group's heads, and
// cut into 8 contiguous chunks, one per XCD (workgroup b runs on XCD b % 8),
// so an XCD's L2 serves neighbouring rows of one KV group.  Each chunk is a
// queue (a counter in the workspace, zeroed by the V^T pre-pass): a
// workgroup takes its XCD's next item, and once that chunk is exhausted it
// takes items of the other chunks.  The XCDs of one part do not run at one
// speed (up to 6 % apart on identical work), and with one item per
// workgroup, dispatched round-robin over the XCDs, the fast ones idled for
// up to 1.5 ms at the end of a 33 ms call; a workgroup also no longer pays a
// dispatch per item.  The next item's counter is bumped when an item starts,
// and the item resolves it into the next item (thread 0 writes it to LDS)
// later on (the bf16 kernel after its first step, the fp8 kernel at the
// barrier that ends its block loop), so the atomic's latency hides under the
// item and the item's end needs no barrier of its own.
// The persistent item loop shared by the attention kernels: runs
// item(i, claim) for every item i in [0, n) that this workgroup claims.  The
// item calls claim() once, with every thread, after one of its barriers and
// before its last one: the barrier before it orders every wave's read of the
// current next_item ahead of the write, the one after it publishes the write.
template <typename F>
__device__ __forceinline__ void run_items(int n, int32_t *ctr, F &&item) {
  __shared__ int32_t next_item;
  const int per = (n + 7) >> 3, xcd = blockIdx.x & 7;
  auto lo_of = [&](int x) { return x * per; };
  auto hi_of = [&](int x) { const int h = (x + 1) * per; return h < n ? h : n; };
  // an item of another chunk, or -1 when every chunk is exhausted (thread 0)
  auto steal = [&]() {
    for (int k = 1; k < 8; ++k) {
      const int x = (xcd + k) & 7, lo = lo_of(x), hi = hi_of(x);
      if (lo >= hi || __hip_atomic_load(&ctr[x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= hi - lo) continue;
      const int i = atomicAdd(&ctr[x], 1);
      if (lo + i < hi) return lo + i;
    }
    return -1;
  };
  auto own_or_steal = [&](int i) { return lo_of(xcd) + i < hi_of(xcd) ? lo_of(xcd) + i : steal(); };
  if (threadIdx.x == 0) next_item = own_or_steal(atomicAdd(&ctr[xcd], 1));
  __syncthreads();
  int cur = next_item;
  // Declared outside the loop: a fresh zero at the top of each item would be
  // a write to the register the previous claim's atomic returns into, which
  // the compiler guards with a wait for every outstanding memory operation.
  int pending = 0;
  while (cur >= 0) {
    if (threadIdx.x == 0) pending = atomicAdd(&ctr[xcd], 1);
    item(cur, [&]() __attribute__((always_inline)) {
      if (threadIdx.x == 0) next_item = own_or_steal(pending);
    });
    cur = __builtin_amdgcn_readfirstlane(next_item);
  }
}

template <bool kSparse, bool kPair>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(AttnLaunch a, SeqTable t, int rows, int32_t *ctr) {
  run_items(rows * a.Hq, ctr, [&](int i, auto &&claim) { attn_bf16_item<kSparse, kPair>(a, t, rows, i, claim); });
}

// ====================================================================== fp8
// e4m3 operands with the 32x32x64 fp8 MFMA: Q.K^T in two K=64 steps per key
// tile, P.V in K=64 steps per head-dim tile.  Per-block scales: the q and k
// scales fold into the exponent scale c of the block, the v scale into the
// exponent offset of the weights (softmax_fp8), so no per-element multiply is
// spent on either.  Two kernels: attn_fp8_kernel rounds the weights to e4m3
// (at most 430 < 448, see softmax_fp8) and adds a second e4m3 pass with the
// rounding residual where a block holds a large share of a query's weight;
// attn_fp8_pv16_kernel keeps every weight in fp16 (11 significant bits) and
// runs P.V on the fp16 V^T image, at the price of twice the P.V MFMA time.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// The residual weights of a heavy block, x - e4m3(x): exact in fp32 and at
// most 2^-4 |x| (<= 27 for x <= 430), packed to e4m3 again for a second P.V
// pass; hi + lo leaves a relative error of about 2^-8 per weight.  Residuals
// of weights below 4 fall into e4m3's subnormal range (steps of 2^-9): an
// absolute error below 2^-10, negligible next to the block's largest weight
// (at least 152 whenever it holds the running maximum).
__device__ __forceinline__ uint32_t pack_lo_fp8x4(float a, float b, float c, float d) {
  const uint32_t h = pack_fp8x4(a, b, c, d);
  const auto ab = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, false);
  const auto cd = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, true);
  return pack_fp8x4(a - ab[0], b - ab[1], c - cd[0], d - cd[1]);
}

// e4m3 x e4m3 with an E8M0 block scale on the B operand (127 = 2^0).
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64_bs(i32x8 a, i32x8 b, f32x16 c, int bscale) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, bscale);
}


template <bool kSparse, typename Claim>
__device__ __forceinline__ void attn_fp8_pv16_item(const AttnLaunch &a, const SeqTable &t, int rows, int item,
                                                   Claim &&claim) {
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[kTile8];      // e4m3 K, [key][d], padded rows
  __shared__ __attribute__((aligned(1024))) uint16_t Vh[kTile16];    // fp16 V^T image (P.V; output staging)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 5, l32 = lane & 31;
  const AttnItem w = decode_item(a, t, rows, item);
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
    block_sync();
    claim();
    block_sync();
    return;
  }
  auto clampJ = [&](int x) { return x < 0 ? 0 : (x > w.I ? w.I : x); };
  // Where K of block J starts: its page when K/V are paged (clamped into the
  // pool), else its packed row.  Scales are always indexed by row: for paged
  // K/V the pre-pass copies each page's scales to row-indexed arrays.
  cint32 *ptab = a.table ? as_const(a.table) + (size_t)(t.z0 + w.z) * a.table_stride : nullptr;
  auto srow = [&](int J) {
    if (!ptab) return zrow + J;
    const int pg = ptab[J];
    return pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
  };

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

  // Direct loads as in the bf16 kernel.  An fp8 tile is 18 instructions
  // (slot s = 64 k + lane holds chunk s % 9 of row s / 9; chunk 8 is the pad),
  // 5 for waves 0-1 and 4 for waves 2-3; the fp16 V^T image is 34.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int nk8 = wv < 2 ? 5 : 4, nk16 = wv < 2 ? 9 : 8;
  const size_t kstride = (size_t)a.Hkv * kHeadDim;
  uint32_t koff[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int sl = 64 * (wv + 4 * m) + lane;
    const int r = sl / 9, ch = sl - 9 * (sl / 9);
    koff[m] = (uint32_t)(r * kstride + 16 * (ch < 8 ? ch : 0));
  }
  const uint8_t *kbase = kp + (size_t)w.g * kHeadDim;
  const uint16_t *v16base = a.vimg16 + ((size_t)w.g * a.R + zrow) * kTile16 + lane * 8;
  auto issue_k = [&](int J) __attribute__((always_inline)) {
    const uint8_t *src = kbase + (size_t)srow(J) * kBlock * kstride;
#pragma unroll
    for (int m = 0; m < 5; ++m)
      if (m < nk8) __builtin_amdgcn_global_load_lds(src + koff[m], lds_ptr(Ks + (wv + 4 * m) * 1024), 16, 0, 0);
  };
  auto issue_v16 = [&](int J) __attribute__((always_inline)) {
    const uint16_t *src = v16base + (size_t)J * kTile16;
#pragma unroll
    for (int m = 0; m < 9; ++m)
      if (m < nk16)
        __builtin_amdgcn_global_load_lds(src + (wv + 4 * m) * 512, lds_ptr(Vh + (wv + 4 * m) * 512), 16, 0, 0);
  };
  // Operand reads: 32 bytes = chunks 4 k + 2 lg and +1 of row 32 t + l32.
  const uint8_t *k8ad = &Ks[l32 * kRow8 + 32 * lg];
  const uint16_t *vhad = &Vh[l32 * kRow16 + 8 * lg];
  auto ld32 = [](const uint8_t *p) __attribute__((always_inline)) {
    const u32x4 lo = ld16(p), hi = ld16(p + 16);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  float R = -INFINITY, L = 0.f;      // softmax_fp8's reference and weight sum
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};

  // One step per listed block J: K of J is in flight when it starts.  The
  // first barrier publishes K of J and marks every wave's P.V of the previous
  // block done, so the fp16 V^T image of J is requested there and lands
  // during Q.K^T and the softmax; the second barrier publishes it and frees
  // the K tile for the next block's K, which lands during P.V.
  //
  // The k and v scales of a block are read one step ahead by scalar loads
  // issued between that step's Q.K^T and its softmax, which waits on no LDS
  // operation: their latency hides under the exponentials.  (Plain loads in
  // the step itself made the first wait on them also wait for its V tile.)
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat *ksc_c = (cfloat *)a.k_scale + (size_t)zrow * a.Hkv + w.g;
  cfloat *vsc_c = (cfloat *)a.v_scale + (size_t)zrow * a.Hkv + w.g;
  float ksc, vsc;                    // scales of the current block
  // kDiag: the diagonal block (causal mask; always a row's last block).  Otherwise has_next says whether a next block Jn follows.
  auto step = [&](auto kDiag, int J, int Jn, bool has_next) __attribute__((always_inline)) {
    constexpr bool diag = decltype(kDiag)::value;
    wait_vmcnt<0>();
    block_sync();
    issue_v16(J);
    const float c = cq * ksc;
    // a zero V scale (an all-zero block) is taken as 2^-64: its weights still
    // count in L, and its codes contribute nothing measurable
    const float vs = fmaxf(vsc, 0x1p-64f);
    f32x16 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        s[tt] = mfma_fp8_32x32x64(ld32(k8ad + 32 * kRow8 * tt + 64 * ks), qf[ks], s[tt]);
    }
    if (has_next) {
      ksc = ksc_c[(size_t)Jn * a.Hkv];
      vsc = vsc_c[(size_t)Jn * a.Hkv];
    }
    softmax_fp8(s, diag, qloc, lg, c, __builtin_amdgcn_logf(vs), __builtin_amdgcn_rcpf(vs), R, L, o);
    wait_vmcnt<0>();
    block_sync();
    if (has_next) issue_k(Jn);
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const int tt = cc >> 1, j0 = 8 * (cc & 1);
      const u32x4 v4 = {pack_f16x2(s[tt][j0 + 0], s[tt][j0 + 1]), pack_f16x2(s[tt][j0 + 2], s[tt][j0 + 3]),
                        pack_f16x2(s[tt][j0 + 4], s[tt][j0 + 5]), pack_f16x2(s[tt][j0 + 6], s[tt][j0 + 7])};
      const f16x8 pk = as_f16x8(v4);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        o[u] = mfma_f16_32x32x16(as_f16x8(ld16(vhad + 32 * kRow16 * u + 16 * cc)), pk, o[u]);
    }
  };

  // Lists are ascending, so only the last block can be the diagonal one:
  // the loop runs every other block (a last block that is not diagonal
  // included, with no next K to request), the diagonal block runs last.
  int J = kSparse ? clampJ(list[0]) : 0;
  issue_k(J);
  ksc = ksc_c[(size_t)J * a.Hkv];
  vsc = vsc_c[(size_t)J * a.Hkv];
  const int last = kSparse ? clampJ(list[n_blk - 1]) : w.I;
  const int n_loop = last == w.I ? n_blk - 1 : n_blk;
  using NotDiag = std::integral_constant<bool, false>;
  using Diag = std::integral_constant<bool, true>;
  for (int b = 0; b < n_loop; ++b) {
    const bool has_next = b + 1 < n_blk;
    const int Jn = has_next ? (kSparse ? clampJ(list[b + 1]) : b + 1) : 0;
    step(NotDiag{}, J, Jn, has_next);
    J = Jn;
  }
  if (n_loop < n_blk) step(Diag{}, J, 0, false);

  const float l_tot = L + __shfl_xor(L, 32, 64);
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[u][i] *= inv;
  block_sync();                      // every wave's last P.V has read Vh
  claim();
  stage_out(Vh, o, qloc, lg);
  if (lse && lg == 0) *lse = (R - kFp8Off + __log2f(l_tot)) * 0.69314718055994531f;
  block_sync();
  store_staged<256>(Vh, (__bf16 *)a.out + (qtok0 * a.Hq + w.h) * kHeadDim, a.Hq, tid);
}

// e4m3 weights: four waves of 32 queries each, three workgroups per CU.  A
// block's S^T is computed, turned into weights and multiplied into O one
// 64-key half at a time, so only 32 logits per lane are live and a wave fits
// in 168 registers (three waves per SIMD).  A half that is heavy for any
// query of the wave (heavy_block), and every half of the diagonal block, gets
// a second e4m3 P.V pass with the rounding residual of its weights
// (pack_lo_fp8x4): its weights then carry about 2^-8 relative error instead
// of 2^-4.  On spread-out attention this is the first few blocks of a row at
// most; on concentrated attention it is the blocks that hold the row's
// weight.  V^T is held in LDS as its two key halves, each [128 d][64 keys]
// with 80-byte rows, so that one half can be loaded while the other is in
// use.  Per block J: barrier (K and V^T half 0 of J landed), load V^T half 1
// of J; half 0: Q.K^T, softmax, P.V; Q.K^T of half 1; barrier (V^T half 1
// landed, every wave done with K and V^T half 0), load K and V^T half 0 of
// the next block; softmax and P.V of half 1.  The k and v scales of the next
// block are read by scalar loads one step ahead.
constexpr int kRowV = 80;                       // bytes of one d row of a V^T half in LDS
constexpr int kHalfV8 = kHeadDim * kRowV;       // 10240 bytes
template <bool kSparse, typename Claim>
__device__ __forceinline__ void attn_fp8_item(const AttnLaunch &a, const SeqTable &t, int rows, int item,
                                               Claim &&claim) {
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[kTile8];       // e4m3 K, [key][d], padded rows
  __shared__ __attribute__((aligned(1024))) uint8_t Vs[2 * kHalfV8];  // e4m3 V^T halves

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 5, l32 = lane & 31;
  const AttnItem w = decode_item(a, t, rows, item);
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
    block_sync();
    claim();
    block_sync();
    return;
  }
  auto clampJ = [&](int x) { return x < 0 ? 0 : (x > w.I ? w.I : x); };
  cint32 *ptab = a.table ? as_const(a.table) + (size_t)(t.z0 + w.z) * a.table_stride : nullptr;
  auto srow = [&](int J) {
    if (!ptab) return zrow + J;
    const int pg = ptab[J];
    return pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
  };

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

  // K tile: 1152 chunks of 16 bytes ([key][9 chunks], the ninth is padding),
  // one chunk per lane and instruction, waves 0-1 five instructions, 2-3 four.
  // V^T half: 640 chunks ([d][5 chunks], the fifth padding) from the image's
  // [d][9 chunks] rows, waves 0-1 three instructions, 2-3 two.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int nk8 = wv < 2 ? 5 : 4, nv8 = wv < 2 ? 3 : 2;
  const uint32_t kstride = (uint32_t)a.Hkv * kHeadDim;
  uint32_t koff[5], voff[3];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const uint32_t sl = 64 * (wv + 4 * m) + lane;
    const uint32_t r = sl / 9, ch = sl - 9 * r;
    koff[m] = r * kstride + 16 * (ch < 8 ? ch : 0);
  }
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const uint32_t sl = 64 * (wv + 4 * m) + lane;
    const uint32_t r = sl / 5, ch = sl - 5 * r;
    voff[m] = r * kRow8 + 16 * (ch < 4 ? ch : 0);
  }
  const uint8_t *kbase = kp + (size_t)w.g * kHeadDim;
  const uint8_t *v8base = a.vimg8 + ((size_t)w.g * a.R + zrow) * kTile8;
  // buffer descriptors over one block (uniform, in SGPRs) take the per-lane
  // offsets as 32-bit values
  auto issue_k = [&](int J) __attribute__((always_inline)) {
    const int pg = __builtin_amdgcn_readfirstlane(srow(J));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(kbase + (size_t)pg * kBlock * kstride), (short)0, (int)(kBlock * kstride), kBufWord3);
#pragma unroll
    for (int m = 0; m < 5; ++m)
      if (m < nk8) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(Ks + (wv + 4 * m) * 1024), 16, koff[m], 0, 0, 0);
  };
  auto issue_vh = [&](int J, int hh) __attribute__((always_inline)) {
    J = __builtin_amdgcn_readfirstlane(J);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(v8base + (size_t)J * kTile8 + 64 * hh), (short)0, kTile8 - 64 * hh, kBufWord3);
#pragma unroll
    for (int m = 0; m < 3; ++m)
      if (m < nv8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(Vs + hh * kHalfV8 + (wv + 4 * m) * 1024), 16, voff[m], 0,
                                                 0, 0);
  };
  const int krow = l32 * kRow8 + 32 * lg, vrow = l32 * kRowV + 32 * lg;
  auto ld32 = [](const uint8_t *p) __attribute__((always_inline)) {
    const u32x4 lo = ld16(p), hi = ld16(p + 16);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  // lanes l and l ^ 32 hold the two key groups of one query: v_permlane32_swap
  // pairs them without an LDS round trip; both lanes get the same result
  auto pair_max = [](float x) __attribute__((always_inline)) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto pair_sum = [](float x) __attribute__((always_inline)) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };

  float R = -INFINITY, L = 0.f;      // reference and weight sum, as in softmax_fp8
  f32x16 o[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) o[u] = f32x16{};

  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat *ksc_c = (cfloat *)a.k_scale + (size_t)zrow * a.Hkv + w.g;
  cfloat *vsc_c = (cfloat *)a.v_scale + (size_t)zrow * a.Hkv + w.g;
  float ksc, vsc;

  // S^T of half h (keys 64 h .. 64 h + 63) for this wave's 32 queries
  auto qk = [&](int h, f32x16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int aa = 0; aa < 2; ++aa) {
      s[aa] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        s[aa] = mfma_fp8_32x32x64(ld32(Ks + krow + 32 * kRow8 * (2 * h + aa) + 64 * ks), qf[ks], s[aa]);
      __builtin_amdgcn_sched_barrier(0);   // one tile's operands in registers at a time
    }
  };
  // softmax of half h and its P.V (plus the residual pass when heavy)
  auto sm_pv = [&](auto kDiag, int h, f32x16 (&s)[2], float c, float lv, float inv_vs)
                   __attribute__((always_inline)) {
    constexpr bool diag = decltype(kDiag)::value;
    if constexpr (diag) {
      const int lim = qloc - 4 * lg - 64 * h;   // key > qloc  <=>  (key - 64 h - 4 lg) > lim
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[aa][i] = (32 * aa + 8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : s[aa][i];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[aa][i]);
    // in the diagonal block a query may see no key of half 1 (cm = -inf: its
    // weights there are 0); it always sees key 0 of half 0, so R is finite
    // from a row's first half on
    const float cm = pair_max(mx) * c;
    const float mz = cm + lv;
    if (__any(mz > R + kFp8Lazy)) {
      const float Rn = fmaxf(R, mz);
      const float f = __builtin_amdgcn_exp2f(R - Rn);   // 0 on the first half (R = -inf), else <= 1
      R = Rn;
      L *= f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[u][i] *= f;
    }
    const float off = lv - R + kFp8Off;
    float psum = 0.f;
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[aa][i], c, off));
        s[aa][i] = p;
        psum += p;
      }
    L = fmaf(psum, inv_vs, L);
    i32x8 pk;
#pragma unroll
    for (int aa = 0; aa < 2; ++aa)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pk[4 * aa + j] = (int)pack_fp8x4(s[aa][4 * j + 0], s[aa][4 * j + 1], s[aa][4 * j + 2], s[aa][4 * j + 3]);
    // the residual (when heavy) is packed before the P.V so that the
    // logits are dead during it
    const bool heavy = diag || __any(heavy_block(cm, R, pair_sum(L)));
    i32x8 pl;
    if (heavy) {
#pragma unroll
      for (int aa = 0; aa < 2; ++aa)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          pl[4 * aa + j] =
              (int)pack_lo_fp8x4(s[aa][4 * j + 0], s[aa][4 * j + 1], s[aa][4 * j + 2], s[aa][4 * j + 3]);
    }
    const uint8_t *vh = Vs + h * kHalfV8 + vrow;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = mfma_fp8_32x32x64_bs(ld32(vh + 32 * kRowV * u), pk, o[u], 127);
    if (heavy) {
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = mfma_fp8_32x32x64_bs(ld32(vh + 32 * kRowV * u), pl, o[u], 127);
    }
  };

  auto step = [&](auto kDiag, int J, int Jn, bool has_next) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    block_sync();                    // K and V^T half 0 of J have landed; every wave is done with V^T half 1
    issue_vh(J, 1);
    const float c = cq * ksc;
    // a zero V scale (an all-zero block) is taken as 2^-64, as in attn_fp8_pv16_item
    const float vs = fmaxf(vsc, 0x1p-64f);
    const float lv = __builtin_amdgcn_logf(vs), inv_vs = __builtin_amdgcn_rcpf(vs);
    if (has_next) {
      ksc = ksc_c[(size_t)Jn * a.Hkv];
      vsc = vsc_c[(size_t)Jn * a.Hkv];
    }
    f32x16 s[2];
    qk(0, s);
    sm_pv(kDiag, 0, s, c, lv, inv_vs);
    qk(1, s);
    wait_vmcnt<0>();
    block_sync();                    // V^T half 1 of J has landed; every wave is done with K and V^T half 0
    if (has_next) {
      issue_k(Jn);
      issue_vh(Jn, 0);
    }
    sm_pv(kDiag, 1, s, c, lv, inv_vs);
  };

  int J = kSparse ? clampJ(list[0]) : 0;
  issue_k(J);
  issue_vh(J, 0);
  ksc = ksc_c[(size_t)J * a.Hkv];
  vsc = vsc_c[(size_t)J * a.Hkv];
  const int last = kSparse ? clampJ(list[n_blk - 1]) : w.I;
  const int n_loop = last == w.I ? n_blk - 1 : n_blk;
  using NotDiag = std::integral_constant<bool, false>;
  using Diag = std::integral_constant<bool, true>;
  for (int b = 0; b < n_loop; ++b) {
    const bool has_next = b + 1 < n_blk;
    const int Jn = has_next ? (kSparse ? clampJ(list[b + 1]) : b + 1) : 0;
    step(NotDiag{}, J, Jn, has_next);
    J = Jn;
  }
  if (n_loop < n_blk) step(Diag{}, J, 0, false);

  const float l_tot = pair_sum(L);
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[u][i] *= inv;
  block_sync();                      // every wave's last P.V has read Vs
  claim();
  // output staging: rows 0-63 in Ks, 64-127 in Vs (64 rows of 272 bytes fit
  // in each).  The lane index is taken afresh here so that the addresses
  // below are not computed before the item loop and held in registers
  // through it.
  int tid_o = tid;
  asm volatile("" : "+v"(tid_o));
  const int lane_o = tid_o & 63, qloc_o = (tid_o >> 6) * 32 + (lane_o & 31);
  uint16_t *stg = (uint16_t *)(wave < 2 ? Ks : Vs) - (wave < 2 ? 0 : 64 * kOutRow);
  stage_out(stg, o, qloc_o, lane_o >> 5);
  if (lse && lg == 0) *lse = (R - kFp8Off + __log2f(l_tot)) * 0.69314718055994531f;
  block_sync();
#pragma unroll
  for (int it = 0; it < kBlock * 16 / 256; ++it) {
    const int cidx = it * 256 + tid_o, row = cidx >> 4, ch = cidx & 15;
    const uint16_t *src = (const uint16_t *)(row < 64 ? Ks : Vs) + (row & 63) * kOutRow + 8 * ch;
    st16((__bf16 *)a.out + ((qtok0 + row) * a.Hq + w.h) * kHeadDim + 8 * ch, ld16(src));
  }
  block_sync();                      // the next item's first loads overwrite the staging
}

// Both fp8 kernels are persistent like the bf16 kernel (run_items): three
// workgroups per CU for e4m3 weights, two for fp16 weights.
template <bool kSparse>
__global__ __launch_bounds__(256, 3) void attn_fp8_kernel(AttnLaunch a, SeqTable t, int rows, int32_t *ctr) {
  run_items(rows * a.Hq, ctr, [&](int i, auto &&claim) { attn_fp8_item<kSparse>(a, t, rows, i, claim); });
}

template <bool kSparse>
__global__ __launch_bounds__(256, 2) void attn_fp8_pv16_kernel(AttnLaunch a, SeqTable t, int rows, int32_t *ctr) {
  run_items(rows * a.Hq, ctr, [&](int i, auto &&claim) { attn_fp8_pv16_item<kSparse>(a, t, rows, i, claim); });
}

// ================================================================ launchers
size_t attn_workspace_ctr_offset(int Hkv, int R, bool fp8) {
  const size_t b = fp8 ? attn_workspace_scales_offset(Hkv, R) + 2 * (size_t)Hkv * R * sizeof(float)
                       : (size_t)Hkv * R * 2 * (size_t)kTile16;
  return (b + 255) / 256 * 256;
}
size_t attn_workspace_bytes(int Hkv, int R, bool fp8, int num_seqs) {
  const size_t launches = (size_t)(num_seqs + kMaxSeqsPerLaunch - 1) / kMaxSeqsPerLaunch;
  return attn_workspace_ctr_offset(Hkv, R, fp8) + (launches * 8 * sizeof(int32_t) + 255) / 256 * 256;
}
size_t attn_workspace_img16_offset(int Hkv, int R) { return (size_t)Hkv * R * kTile8; }
size_t attn_workspace_scales_offset(int Hkv, int R) {
  return (size_t)Hkv * R * ((size_t)kTile8 + 2 * (size_t)kTile16);
}

hipError_t launch_vprep(const AttnLaunch &a, bool fp8, hipStream_t s) {
  const dim3 grid(a.R, a.Hkv);
  if (fp8)
    hipLaunchKernelGGL(vprep_fp8_kernel, grid, dim3(256), 0, s, (const uint8_t *)a.v, a.vimg8, a.vimg16,
                       a.Hkv, a.R, a.ctr, a.n_ctr);
  else
    hipLaunchKernelGGL(vprep_bf16_kernel, grid, dim3(256), 0, s, (const __bf16 *)a.v, a.vimg16, a.Hkv, a.R, a.ctr,
                       a.n_ctr);
  return hipGetLastError();
}

hipError_t launch_vprep_paged(const AttnLaunch &a, const SeqTable &t, int rows, int launch_index, hipStream_t s) {
  const dim3 grid(rows, a.Hkv);
  hipLaunchKernelGGL(vprep_fp8_paged_kernel, grid, dim3(256), 0, s, (const uint8_t *)a.v, a.vimg8, a.vimg16, a.Hkv,
                     a.R, a.table, a.table_stride, a.num_pages, t, a.k_scale_pages, a.v_scale_pages,
                     (float *)a.k_scale, (float *)a.v_scale, a.ctr + 8 * launch_index);
  return hipGetLastError();
}

// Workgroups of a persistent attention kernel: per_cu per CU of the stream's
// device (no more than there are items).
static int persistent_grid(hipStream_t s, int n_items, int per_cu) {
  int dev = 0;
  if (s) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(s, &d) == hipSuccess) dev = (int)d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    dev = 0;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  return n_items < cus * per_cu ? n_items : cus * per_cu;
}

hipError_t launch_attn(const AttnLaunch &a, const SeqTable &t, int rows, bool sparse, bool fp8, bool pv16,
                       int launch_index, hipStream_t s) {
  int32_t *ctr = a.ctr + 8 * launch_index;
  if (fp8) {
    if (pv16) {
      const dim3 pgrid(persistent_grid(s, rows * a.Hq, 2));
      if (sparse) hipLaunchKernelGGL((attn_fp8_pv16_kernel<true>), pgrid, dim3(256), 0, s, a, t, rows, ctr);
      else hipLaunchKernelGGL((attn_fp8_pv16_kernel<false>), pgrid, dim3(256), 0, s, a, t, rows, ctr);
    } else {
      const dim3 pgrid(persistent_grid(s, rows * a.Hq, 3));
      if (sparse) hipLaunchKernelGGL((attn_fp8_kernel<true>), pgrid, dim3(256), 0, s, a, t, rows, ctr);
      else hipLaunchKernelGGL((attn_fp8_kernel<false>), pgrid, dim3(256), 0, s, a, t, rows, ctr);
    }
  } else {
    const dim3 pgrid(persistent_grid(s, rows * a.Hq, 1));
    if (sparse) hipLaunchKernelGGL((attn_bf16_kernel<true, false>), pgrid, dim3(512), 0, s, a, t, rows, ctr);
    else hipLaunchKernelGGL((attn_bf16_kernel<false, false>), pgrid, dim3(512), 0, s, a, t, rows, ctr);
  }
  return hipGetLastError();
}

hipError_t launch_attn_q64(const AttnLaunch &a, const SeqTable &t, int rows, int launch_index, hipStream_t s) {
  const dim3 pgrid(persistent_grid(s, rows * a.Hq, 1));
  hipLaunchKernelGGL((attn_bf16_kernel<true, true>), pgrid, dim3(512), 0, s, a, t, rows, a.ctr + 8 * launch_index);
  return hipGetLastError();
}

}  // namespace stem
