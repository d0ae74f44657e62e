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

// fp8: writes the e4m3 V^T image (16 KB per block) and an fp16 V^T image
// (32 KB per block, exact) used when the block is a row's diagonal block.
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
                                                        uint16_t *__restrict__ img16, int Hkv, int R) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kBlock * (kHeadDim + 16)];
  const int kb = blockIdx.x, g = blockIdx.y;
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
                                                              float *__restrict__ ksr, float *__restrict__ vsr) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kBlock * (kHeadDim + 16)];
  const int kb = t.row[0] + blockIdx.x, g = blockIdx.y;
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
__device__ __forceinline__ AttnItem decode_attn(const AttnLaunch &a, const SeqTable &t, int rows) {
  const int G = a.Hq / a.Hkv;
  const int item = xcd_chunk_item(blockIdx.x, rows * a.Hq);
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
// range as far down as with P' = 256 p.  O is rarely touched.  Leaves P' in s.
constexpr float kFp8Lazy = 0.75f;
constexpr float kFp8Off = 8.f;
__device__ __forceinline__ void softmax_fp8(f32x16 (&s)[4], bool diag, int qloc, int lg, float c, float lv,
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
  // itself in the diagonal one), so mz is finite
  const float mz = fmaf(wave_max_xor32(mx), c, lv);
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
}

// ===================================================================== bf16
// One workgroup of 8 waves per (query head, query block), one workgroup per
// CU.  Waves w and w + 4 share a SIMD and the same 32 queries (w & 3); wave w
// (group 0) takes keys 0-63 of every listed block, wave w + 4 (group 1) keys
// 64-127, each with its own online softmax, merged once per row.  A group
// loads only its own halves of the K and V^T tiles.
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
// two lists, and a block that is not in a half's list gets zero weight for
// that half's queries.  Waves qw = 0, 1 hold half 0 and qw = 2, 3 half 1, so
// the test is wave-uniform and such a wave skips its softmax.  The union is
// built once per workgroup in LDS (a bitmap per half, then one wave compacts
// their OR in ascending order), so the block loop is the square-row loop.  On gfx950
// this costs the same per listed block as square rows (measured equal on the
// 128K layer), whereas a 64-query tile halves the MFMA work per K/V tile but
// keeps the tile loads and barriers (measured 2.35x slower).
constexpr float kLazyLog2 = 8.f;
constexpr int kHalfK = 64 * kRow16;              // K half: 64 keys x 17 chunks (elements)
constexpr int kRowVh = 72;                       // V^T half row: 64 keys + pad chunk (elements)
constexpr int kHalfV = kHeadDim * kRowVh;        // V^T half: 128 dims x 9 chunks (elements)
constexpr uint32_t kBufWord3 = 0x00020000u;      // raw buffer descriptor word 3 (gfx9 dword access)

template <bool kSparse, bool kPair>
__global__ __launch_bounds__(512, 1) void attn_bf16_kernel(AttnLaunch a, SeqTable t, int rows) {
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
  const int qw = wv & 3, kh = wv >> 2;
  const AttnItem w = decode_attn(a, t, rows);
  const int zrow = t.row[w.z];
  const size_t ztok = (size_t)t.tok[w.z];
  const size_t qtok0 = ztok + (size_t)w.I * kBlock;
  const int qloc = qw * 32 + l32;
  const size_t qtok = qtok0 + qloc;
  // kPair: list rows 2r (queries 0-63) and 2r + 1 (queries 64-127)
  const size_t lrow = kPair ? ((size_t)w.h * a.R + w.r) * 2 : (size_t)w.h * a.R + w.r;
  cint32 *list = kSparse ? as_const(a.idx) + lrow * a.k_cap : nullptr;
  // Lists are trusted to be ascending in [0, I]; counts and ids are still
  // clamped so a malformed list can never address outside the sequence.
  int n_blk = kSparse ? as_const(a.cnt)[lrow] : w.I + 1;
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
    if (kh == 0) write_empty(orow, lse, lg);
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
  const int my_bit = qw < 2 ? 1 : 2;

  // Q as the B operand: query qloc, head dims 16 ks + 8 lg .. +7
  bf16x8 qf[8];
  {
    const __bf16 *qrow = (const __bf16 *)a.q + (qtok * a.Hq + w.h) * kHeadDim + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(ld16(qrow + 16 * ks));
  }

  // Direct loads through raw buffer descriptors rebased per block (32-bit
  // per-lane offsets, scalar bases).  Load instruction k of a half writes
  // LDS slots 64 k + lane (16 B each); group wave qw issues k = qw + 4 m.
  //   K half: 17 loads; slot s -> key row s / 17, chunk s % 17 (chunk 16 is
  //           the pad and re-reads chunk 0).
  //   V half: 18 loads; slot s -> dim row s / 9, chunk s % 9 of this half's
  //           8 image chunks (chunk 8 is the pad and re-reads chunk 0).
  const uint32_t kstride_b = (uint32_t)a.Hkv * kHeadDim * 2;
  const int nkk = qw == 0 ? 5 : 4, nkv = qw < 2 ? 5 : 4;
  uint32_t koff[5], voff[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const int sk = 64 * (qw + 4 * m) + lane;
    const int rk = sk / 17, ck = sk - 17 * rk;
    koff[m] = (uint32_t)rk * kstride_b + 16 * (ck < 16 ? ck : 0);
    const int sv = 64 * (qw + 4 * m) + lane;
    const int rv = sv / 9, cv = sv - 9 * rv;
    voff[m] = (uint32_t)(rv * kRow16 * 2 + 16 * (8 * kh + (cv < 8 ? cv : 0)));
  }
  const char *kbase = (const char *)a.k + ((ztok + 64 * kh) * a.Hkv + w.g) * kHeadDim * 2;
  const char *vbase = (const char *)(a.vimg16 + ((size_t)w.g * a.R + zrow) * kTile16);
  // Block ids are wave-uniform; readfirstlane keeps the descriptors in SGPRs.
  auto issue_k = [&](int J, uint16_t *Kd) __attribute__((always_inline)) {
    J = __builtin_amdgcn_readfirstlane(J);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(kbase + (size_t)J * kBlock * kstride_b), (short)0, (int)(64 * kstride_b), kBufWord3);
    uint16_t *d = Kd + kh * kHalfK;
#pragma unroll
    for (int m = 0; m < 5; ++m)
      if (m < nkk) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(d + (qw + 4 * m) * 512), 16, koff[m], 0, 0, 0);
  };
  // The loads of one block step: d = 0..4 are K loads m = d of the next
  // block (a descriptor of size 0 when there is none: no memory is read and
  // the free buffer gets zeros), d = 5..9 are V loads m = d - 5 of this block.
  auto k_rsrc = [&](int Jn, bool has_next) __attribute__((always_inline)) {
    Jn = __builtin_amdgcn_readfirstlane(Jn);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(kbase + (size_t)Jn * kBlock * kstride_b), (short)0,
                                             has_next ? (int)(64 * kstride_b) : 0, kBufWord3);
  };
  auto v_rsrc = [&](int J) __attribute__((always_inline)) {
    J = __builtin_amdgcn_readfirstlane(J);
    return __builtin_amdgcn_make_buffer_rsrc((void *)(vbase + (size_t)J * kTile16 * 2), (short)0, kTile16 * 2,
                                             kBufWord3);
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
  auto mfma_phase = [&](auto kPV, const uint16_t *Vp, const uint16_t *Kc, __amdgpu_buffer_rsrc_t rk,
                        __amdgpu_buffer_rsrc_t rv, uint16_t *Kn, uint16_t *Vc) __attribute__((always_inline)) {
    constexpr bool PV = decltype(kPV)::value;
    uint16_t *dk = Kn + kh * kHalfK, *dv = Vc + kh * kHalfV;
    auto dma = [&](int d) __attribute__((always_inline)) {
      if (d < 5) {
        if (d < nkk) __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, lds_ptr(dk + (qw + 4 * d) * 512), 16, koff[d], 0, 0, 0);
      } else {
        const int m = d - 5;
        if (m < nkv) __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, lds_ptr(dv + (qw + 4 * m) * 512), 16, voff[m], 0, 0, 0);
      }
    };
    constexpr int i0 = PV ? 0 : 16;
    const uint16_t *vad = Vp + kh * kHalfV + l32 * kRowVh + 8 * lg;
    const uint16_t *kad = Kc + kh * kHalfK + l32 * kRow16 + 8 * lg;
    auto rd = [&](int i) __attribute__((always_inline)) {
      return i < 16 ? ld16(vad + 32 * kRowVh * (i & 3) + 16 * (i >> 2))
                    : ld16(kad + 32 * kRow16 * ((i - 16) & 1) + 16 * ((i - 16) >> 1));
    };
    u32x4 r[32];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = i0; i < i0 + kAhead; ++i) r[i] = rd(i);
#pragma unroll
    for (int i = i0; i < 32; ++i) {
      if (i + kAhead < 32) r[i + kAhead] = rd(i + kAhead);
      if (PV ? (i % 3 == 1 && i < 30) : (i - 16 < 10)) dma(PV ? i / 3 : i - 16);
      __builtin_amdgcn_sched_barrier(0);
      if (i < 16) {
        o[i & 3] = mfma_f16_32x32x16(as_f16x8(r[i]), as_f16x8(pk[i >> 2]), o[i & 3]);
      } else {
        const int tt = (i - 16) & 1, ks = (i - 16) >> 1;
        s[tt] = mfma_bf16_32x32x16(as_bf16x8(r[i]), qf[ks], ks == 0 ? f32x16{} : s[tt]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // P.V of the last block (no S^T after it).
  auto pv_last = [&](const uint16_t *Vp) __attribute__((always_inline)) {
    const uint16_t *vad = Vp + kh * kHalfV + l32 * kRowVh + 8 * lg;
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
    if (off) {                     // kPair: not in this half's list, zero weight
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) pk[cc] = u32x4{0u, 0u, 0u, 0u};
      return;
    }
    if (diag) {
      const int lim = qloc - 64 * kh - 4 * lg;        // key > qloc  <=>  local key offset > lim
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
  int own = 0;                       // kPair: ownership of the current block in bits 16-17
  auto step = [&](auto kPV, int b, int &J, const uint16_t *Kc, const uint16_t *Vp, uint16_t *Kn, uint16_t *Vc)
                  __attribute__((always_inline)) {
    const int en = b + 1 < n_blk ? blk_entry(b + 1) : 0;
    const int Jn = kPair ? (en & 0xffff) : en;
    wait_vmcnt<0>();                 // this wave's K of b and V of b-1 have landed
    block_sync();                    // ... the whole group's too; Kn and Vc are free
    mfma_phase(kPV, Vp, Kc, k_rsrc(Jn, b + 1 < n_blk), v_rsrc(J), Kn, Vc);
    block_sync();
    softmax(J == w.I, kPair && ((own >> 16) & my_bit) == 0);
    J = Jn;
    own = en;
  };
  using NoPV = std::integral_constant<bool, false>;
  using WithPV = std::integral_constant<bool, true>;

  if constexpr (kPair) own = blk_entry(0);
  int J = blk(0);
  issue_k(J, K0);
  if (kh == 1) block_sync();         // group 1 runs one phase behind
  step(NoPV{}, 0, J, K0, V1, K1, V0);
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
  pv_last((n_blk & 1) ? V0 : V1);
  if (kh == 0) block_sync();         // realign the groups

  // merge the two key halves: waves 4-7 hand (O, m, l) to waves 0-3 through LDS
  block_sync();
  float *xch = (float *)(qw < 2 ? K0 : K1) + (qw & 1) * (66 * 64);
  if (kh == 1) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) xch[(16 * u + i) * 64 + lane] = o[u][i];
    xch[64 * 64 + lane] = m_run;
    xch[65 * 64 + lane] = l_run;
  }
  block_sync();
  if (kh == 0) {
    // the merged max is finite: the key equal to the query is visible in one half
    const float m1 = xch[64 * 64 + lane], l1 = xch[65 * 64 + lane];
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
      for (int i = 0; i < 16; ++i) o[u][i] = (o[u][i] * a0 + xch[(16 * u + i) * 64 + lane] * a1) * inv;
    write_out(orow, o, 1.f, lg);
    if (lse && lg == 0) *lse = kPair && !(l > 0.f) ? -INFINITY : (m + __log2f(l)) * 0.69314718055994531f;
  }
}

// ====================================================================== fp8
// Same pipeline on e4m3 operands with the 32x32x64 fp8 MFMA: Q.K^T in two
// K=64 steps per key tile, P quantised to e4m3 (at most 430 < 448, see
// softmax_fp8), P.V in two K=64 steps per head-dim tile.  Per-block scales:
// the q and k scales fold into the exponent scale c of the block, the v
// scale into the exponent offset of the weights (softmax_fp8), so no
// per-element multiply is spent on either.  The diagonal block, where the
// first queries of a sequence see only a few keys and 3-bit weights would not
// average out, runs its P.V in fp16 from the exact fp16 V^T image.  kPV16
// runs every block's P.V that way (fp16 weights, 11 significant bits): the
// e4m3 V^T tile is then never loaded, and a row whose attention sits on a few
// keys keeps bf16-level accuracy, at the price of twice the P.V MFMA time.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}


template <bool kSparse, bool kPV16>
__global__ __launch_bounds__(256, 2) void attn_fp8_kernel(AttnLaunch a, SeqTable t, int rows) {
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[kTile8];      // e4m3 K, [key][d], padded rows
  __shared__ __attribute__((aligned(1024))) uint8_t Vs[kTile8];      // e4m3 V^T image (unused with kPV16)
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
  // 5 for waves 0-1 and 4 for waves 2-3; the fp16 diagonal image is 34.
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
  const uint8_t *v8base = a.vimg8 + ((size_t)w.g * a.R + zrow) * kTile8 + lane * 16;
  const uint16_t *v16base = a.vimg16 + ((size_t)w.g * a.R + zrow) * kTile16 + lane * 8;
  auto issue_k = [&](int J) __attribute__((always_inline)) {
    const uint8_t *src = kbase + (size_t)srow(J) * kBlock * kstride;
#pragma unroll
    for (int m = 0; m < 5; ++m)
      if (m < nk8) __builtin_amdgcn_global_load_lds(src + koff[m], lds_ptr(Ks + (wv + 4 * m) * 1024), 16, 0, 0);
  };
  auto issue_v8 = [&](int J) __attribute__((always_inline)) {
    const uint8_t *src = v8base + (size_t)J * kTile8;
#pragma unroll
    for (int m = 0; m < 5; ++m)
      if (m < nk8)
        __builtin_amdgcn_global_load_lds(src + (wv + 4 * m) * 1024, lds_ptr(Vs + (wv + 4 * m) * 1024), 16, 0, 0);
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
  const uint8_t *v8ad = &Vs[l32 * kRow8 + 32 * lg];
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
  // block done, so V of J (the fp16 image for the diagonal block or under
  // kPV16, else the e4m3 one) is requested there and lands during Q.K^T and
  // the softmax; the second barrier publishes it and frees the K tile for the
  // next block's K, which lands during P.V.
  auto step = [&](int J, int Jn, bool has_next, bool may_diag) __attribute__((always_inline)) {
    wait_vmcnt<0>();
    block_sync();
    const bool diag = may_diag && (J == w.I);
    if (kPV16 || diag) issue_v16(J); else issue_v8(J);
    const int sr = zrow + J;
    const float c = cq * a.k_scale[(size_t)sr * a.Hkv + w.g];
    const float vs = a.v_scale[(size_t)sr * a.Hkv + w.g];
    f32x16 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        s[tt] = mfma_fp8_32x32x64(ld32(k8ad + 32 * kRow8 * tt + 64 * ks), qf[ks], s[tt]);
    }
    softmax_fp8(s, diag, qloc, lg, c, __builtin_amdgcn_logf(vs), __builtin_amdgcn_rcpf(vs), R, L, o);
    wait_vmcnt<0>();
    block_sync();
    if (has_next) issue_k(Jn);
    if (!kPV16 && !diag) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        i32x8 pk;
#pragma unroll
        for (int aa = 0; aa < 2; ++aa)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x16 &st = s[2 * cc + aa];
            pk[4 * aa + j] = (int)pack_fp8x4(st[4 * j + 0], st[4 * j + 1], st[4 * j + 2], st[4 * j + 3]);
          }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          o[u] = mfma_fp8_32x32x64(ld32(v8ad + 32 * kRow8 * u + 64 * cc), pk, o[u]);
      }
    } else {
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
    }
  };

  // Lists are ascending, so only the last block can be the diagonal one.
  int J = kSparse ? clampJ(list[0]) : 0;
  issue_k(J);
  for (int b = 0; b + 1 < n_blk; ++b) {
    const int Jn = kSparse ? clampJ(list[b + 1]) : b + 1;
    step(J, Jn, true, false);
    J = Jn;
  }
  step(J, 0, false, true);

  const float l_tot = L + __shfl_xor(L, 32, 64);
  write_out(orow, o, 1.f / l_tot, lg);
  if (lse && lg == 0) *lse = (R - kFp8Off + __log2f(l_tot)) * 0.69314718055994531f;
}

// ================================================================ launchers
size_t attn_workspace_bytes(int Hkv, int R, bool fp8) {
  if (!fp8) return (size_t)Hkv * R * 2 * (size_t)kTile16;
  return attn_workspace_scales_offset(Hkv, R) + 2 * (size_t)Hkv * R * sizeof(float);
}
size_t attn_workspace_img16_offset(int Hkv, int R) { return (size_t)Hkv * R * kTile8; }
size_t attn_workspace_scales_offset(int Hkv, int R) {
  return (size_t)Hkv * R * ((size_t)kTile8 + 2 * (size_t)kTile16);
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

hipError_t launch_vprep_paged(const AttnLaunch &a, const SeqTable &t, int rows, hipStream_t s) {
  const dim3 grid(rows, a.Hkv);
  hipLaunchKernelGGL(vprep_fp8_paged_kernel, grid, dim3(256), 0, s, (const uint8_t *)a.v, a.vimg8, a.vimg16, a.Hkv,
                     a.R, a.table, a.table_stride, a.num_pages, t, a.k_scale_pages, a.v_scale_pages,
                     (float *)a.k_scale, (float *)a.v_scale);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnLaunch &a, const SeqTable &t, int rows, bool sparse, bool fp8, bool pv16,
                       hipStream_t s) {
  const dim3 grid(rows * a.Hq);
  if (fp8 && pv16) {
    if (sparse) hipLaunchKernelGGL((attn_fp8_kernel<true, true>), grid, dim3(256), 0, s, a, t, rows);
    else hipLaunchKernelGGL((attn_fp8_kernel<false, true>), grid, dim3(256), 0, s, a, t, rows);
  } else if (fp8) {
    if (sparse) hipLaunchKernelGGL((attn_fp8_kernel<true, false>), grid, dim3(256), 0, s, a, t, rows);
    else hipLaunchKernelGGL((attn_fp8_kernel<false, false>), grid, dim3(256), 0, s, a, t, rows);
  } else {
    if (sparse) hipLaunchKernelGGL((attn_bf16_kernel<true, false>), grid, dim3(512), 0, s, a, t, rows);
    else hipLaunchKernelGGL((attn_bf16_kernel<false, false>), grid, dim3(512), 0, s, a, t, rows);
  }
  return hipGetLastError();
}

hipError_t launch_attn_q64(const AttnLaunch &a, const SeqTable &t, int rows, hipStream_t s) {
  const dim3 grid(rows * a.Hq);
  hipLaunchKernelGGL((attn_bf16_kernel<true, true>), grid, dim3(512), 0, s, a, t, rows);
  return hipGetLastError();
}

}  // namespace stem
