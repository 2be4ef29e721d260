// HIP kernels (gfx950 / CDNA4) for the linear-memory attention-relation KL of LinearARD.
//
// Method: pith.science verdict page on LinearARD (pith_extraction.key_machinery,
// core_discovery): per head, R_m = softmax(scale * X_m X_m^T + M) for teacher and
// student, row-wise forward KL(R_t || R_s); phase 1 keeps only per-row log-sum-exp
// statistics; the backward recomputes logits tile by tile and uses the identity
// dL/dZ_s = g * (R_s - R_t).  The arXiv abstract (mlsanity.com) states that the kernel
// fuses the logit recomputation into the backward and is exact.
//
// Layout of the work:
//  * Forward: a workgroup of 4 wave64s owns a row tile of 128 consecutive rows i of one
//    (batch, head) unit, 32 per wave; two workgroups share a CU, so every SIMD runs two
//    waves.  Backward: a workgroup of 8 waves (two per SIMD) owns 256 rows.  Each wave keeps
//    its rows of the teacher and student as MFMA B operands in registers.
//  * Key tiles of 64 rows j are copied global -> LDS by the DMA path
//    (global_load_lds_dwordx4), double-buffered in the forward and triple-buffered in the
//    backward, one barrier per tile.  LDS rows are unpadded; their 16-byte chunks are
//    XOR-swizzled by the row so that both the 16-byte fragment reads of the score
//    contraction and the transposed 8-byte reads of the gradient contraction hit distinct
//    banks.  Fragment reads run ahead of their MFMAs (explicit software pipelines).
//  * Score blocks are computed transposed, S^T[j][i] = <X[j], X[i]>, with
//    v_mfma_f32_32x32x16 (fp32 inputs: v_mfma_f32_32x32x2f32), so that a lane holds one
//    row i and 16 of its columns j: row statistics reduce inside the lane, and the
//    probability block is already in the A-operand layout of the gradient contraction.
//  * Forward: one online sweep per row keeps (bias, sum, sum of e_t (S_t - S_s)) for
//    teacher and student; the two half-waves sharing a row merge at the end.  For the
//    relation the diagonal score S_ii = |X_i|^2 is the row's reference: it is computed in
//    fp64 from the row itself, sets the initial bias and is added to the sums exactly at the
//    end, so that the KL of nearly equal rows keeps relative precision.  Outputs are per row
//    only: LSE of both sides, the row KL, and R_s(i,i) - R_t(i,i) for the backward.
//  * Backward: the owner of a row tile sweeps the whole row (all key tiles), forms
//    W = dZ + dZ^T block by block (row statistics below the diagonal, column statistics
//    above it, both on it; the diagonal entry from the forward), carries W * 2^14 as fp16
//    and accumulates W X_s on v_mfma_f32_32x32x16_f16, reading X_s transposed from an fp16
//    image of the staged key tile with ds_read_b64_tr_b16.  The row statistics are the
//    forward's LSE vectors, staged with each key tile.  No atomics: every output row has
//    one owner (times an optional split over key tiles reduced in a fixed order).

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <array>
#include <type_traits>
#include <utility>

#include "relkl_internal.h"

namespace lard {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for masked logits
constexpr float kPosBig = 1.0e30f;   // statistic of rows beyond N (probabilities become 0)
constexpr float kWScaleLog2 = 14.0f;  // W is carried as W * 2^14 through fp16
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ element traits
// A "fragment" is 8 consecutive elements along d of one row: the k-chunk one lane
// supplies to a 16-deep step of the score contraction.  frag_t is the score operand type,
// gfrag_t the type of the gradient contraction's operands (the staged student rows and W).
struct Bf16In {  // bf16 inputs (forward)
  using elem_t = uint16_t;
  using frag_t = bf16x8;
  using gfrag_t = bf16x8;
  static constexpr int kES = 2;
  static constexpr bool kConvert = false;
};
struct Bf16Op {  // bf16 inputs in the backward: scores on the bf16 rows as given, the
                 // gradient on an IEEE fp16 image of each staged student tile, made in LDS
  using elem_t = uint16_t;
  using frag_t = bf16x8;
  using gfrag_t = f16x8;
  static constexpr int kES = 2;
  static constexpr bool kConvert = true;
};
struct F16Op {   // fp16 images of bf16 values (the cross relation's reserve copies)
  using elem_t = uint16_t;
  using frag_t = f16x8;
  using gfrag_t = f16x8;
  static constexpr int kES = 2;
  static constexpr bool kConvert = false;
};
struct F32In {   // fp32 inputs (forward and backward)
  using elem_t = float;
  using frag_t = f32x8;
  using gfrag_t = f32x8;
  static constexpr int kES = 4;
  static constexpr bool kConvert = false;
};

__device__ __forceinline__ f32x16 mma_k16(const bf16x8& a, const bf16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mma_k16(const f16x8& a, const f16x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// fp32: eight k=2 steps; in step q a lane of half h supplies k-slot h with its element q,
// the same (h, q) -> k assignment for both operands, so the 16 k values are each summed
// exactly once.
__device__ __forceinline__ f32x16 mma_k16(const f32x8& a, const f32x8& b, f32x16 c) {
#pragma unroll
  for (int q = 0; q < 8; ++q) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], c, 0, 0, 0);
  return c;
}

template <class In>
__device__ __forceinline__ typename In::frag_t load_frag_global(const typename In::elem_t* p) {
  if constexpr (In::kES == 2) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    return __builtin_bit_cast(typename In::frag_t, v);
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Map the hardware workgroup index to a work index such that the workgroups the
// dispatcher sends to one XCD (consecutive g with equal g % 8) get consecutive work
// items: neighbouring row tiles of one unit then share key tiles in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int g, int G) {
  const int full = G & ~7;
  if (g >= full) return g;
  return (g & 7) * (full >> 3) + (g >> 3);
}

// Member of a grouped launch that workgroup (or block) g belongs to, and g's index
// inside it.  Wave-uniform: a few scalar compares.
template <class M>
__device__ __forceinline__ int member_of(const Launch<M>& L, int g) {
  int k = 0;
#pragma unroll
  for (int q = 0; q < kMaxGroup - 1; ++q) k += (q + 1 < L.n && g >= L.end[q]) ? 1 : 0;
  return k;
}

template <class M>
__device__ __forceinline__ int member_begin(const Launch<M>& L, int k) {
  return k == 0 ? 0 : L.end[k - 1];
}

// Input head of relation head h of a member.
template <class M>
__device__ __forceinline__ int head_of(const Launch<M>& L, int map_off, int h) {
  return map_off < 0 ? h : (int)L.head_map[map_off + h];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Wait for this wave's outstanding vector-memory operations (the LDS DMA included).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(const LDS_AS char*)p;
}

// LDS copy of 16 bytes per lane (lane l writes lds_base + 16 l), issued as inline assembly
// so that the compiler does not track it.  Tracking the copies, the compiler waits for all
// of them before any LDS read it cannot prove disjoint from a copy target (the backward
// picks its stage buffers at run time), and it stops counting LDS reads individually:
// every read then waits for all earlier ones (lgkmcnt(0)), which breaks the read-ahead of
// the matrix pipelines.  Completion is awaited explicitly with wait_vmem() before the
// barrier that publishes a tile.  The s_nop covers the one wait state needed between a
// scalar write of M0 and the copy.  A vector instruction that writes a scalar operand of a
// copy (M0 or the base, e.g. v_readfirstlane) would need five, and the compiler's hazard
// checks do not look inside the asm: the compiled kernels are checked statically to have no
// such write that close to a copy (they take their bases and M0 from scalar instructions).
__device__ __forceinline__ void lds_copy16(const void* g, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_base) : "memory");
}

// The same copy from a wave-uniform base address plus a 32-bit per-lane byte offset (the
// scalar-base form: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void lds_copy16_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "{m0}"(lds_base) : "memory");
}

// LDS copy of 4 bytes per lane from a wave-uniform base plus a per-lane byte offset.
__device__ __forceinline__ void lds_copy4_s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
               "{m0}"(lds_base) : "memory");
}

// LDS copy of 4 bytes per lane (lane l writes lds_base + 4 l), as lds_copy16.
__device__ __forceinline__ void lds_copy4(const void* g, uint32_t lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds_base) : "memory");
}

// Workgroup barrier of the backward's tile pipeline.  It completes this wave's LDS reads
// (lgkmcnt(0)) and keeps the compiler from moving memory accesses across it, but unlike
// __syncthreads() it does not wait for the wave's LDS copies still in flight (the fence
// of __syncthreads() waits for every outstanding memory operation).  A copied tile is
// published by an explicit wait_vmem() of every issuing wave before the barrier after
// which it is read.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ LDS key tiles
// Row-major [kBC][D] tile, 16-byte chunks of row r stored at chunk (c ^ swz(r)).  The LDS
// has 64 four-byte banks, i.e. 16 chunk slots per 256-byte bank line.  For rows of 16 or
// more chunks, swz(r) = 4 (r % 4) + (r / 4) % 4 is a bijection on r % 16, so the 16
// rows a 16-byte fragment read touches at one chunk land on 16 distinct slots; and for
// any 4 consecutive rows (aligned to 4) it spreads a run of 4 adjacent chunks over 16
// distinct slots, which is what a transposed 8-byte read of 32 lanes touches.  Rows of 8
// chunks use the 8-slot analogue.
template <int D, int ES>
struct Geo {
  static constexpr int kRowBytes = D * ES;
  static constexpr int kCPR = kRowBytes / 16;  // chunks per row
  static constexpr int kTileBytes = kBC * kRowBytes;
  static constexpr int kDmaPerWave = kBC * kCPR / (kWave * kWaves);
  static_assert(kCPR >= 8, "swizzle needs at least 8 chunks per row");
  static_assert(kBC * kCPR % (kWave * kWaves) == 0, "tile must split evenly over the waves");
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (kCPR >= 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return ((r & 3) << 1) | ((r >> 2) & 1);
  }
  __device__ static __forceinline__ int off(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }
};

// Copy key rows [j0, j0 + kBC) of one unit (row stride `sn_bytes`) into an LDS tile.  Lane
// l of DMA instruction q of wave w fills LDS chunk slot t = (w Q + q) 64 + l (the DMA
// writes lane l at base + 16 l); the slot's row and swizzled chunk say which global
// chunk it takes.  Rows beyond N read row N-1 (finite values, masked by the callers).
template <int D, int ES>
__device__ __forceinline__ void dma_tile(const char* base, int64_t sn_bytes, int j0, int N,
                                         char* lds, int wave, int lane) {
  using G = Geo<D, ES>;
  if (j0 + kBC <= N && sn_bytes < (1 << 24)) {
    // whole tile: a uniform tile base plus per-lane offsets that do not depend on the tile
    const char* tb = base + (int64_t)j0 * sn_bytes;
#pragma unroll
    for (int q = 0; q < G::kDmaPerWave; ++q) {
      const int slot0 = (wave * G::kDmaPerWave + q) * kWave;
      const int t = slot0 + lane;
      const int r = t / G::kCPR;
      const int c = (t % G::kCPR) ^ G::swz(r);
      lds_copy16_s((uint32_t)(r * (int)sn_bytes + c * 16), tb, lds_addr(lds + slot0 * 16));
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < G::kDmaPerWave; ++q) {
    const int slot0 = (wave * G::kDmaPerWave + q) * kWave;
    const int t = slot0 + lane;
    const int r = t / G::kCPR;
    const int c = (t % G::kCPR) ^ G::swz(r);
    const int j = min(j0 + r, N - 1);
    const char* g = base + (int64_t)j * sn_bytes + c * 16;
    lds_copy16(g, lds_addr(lds + slot0 * 16));
  }
}

// Score-contraction A fragment of key row 32 jb + l32, elements 16 ks + 8 hh .. +7.  The
// swizzle of that row only depends on l32 (32 jb is a multiple of 16), and chunk
// 2 ks + hh (2-byte types) or 4 ks + 2 hh (fp32) differs from the ks = 0 chunk by XOR
// with 2 ks (resp. 4 ks): so the address is a per-lane base XOR a constant, plus the
// immediate 32 jb rows.
template <class In, int D>
__device__ __forceinline__ int frag_base(int l32, int hh) {
  using G = Geo<D, In::kES>;
  return In::kES == 2 ? G::off(l32, hh) : G::off(l32, 2 * hh);
}

template <class In, int D>
__device__ __forceinline__ typename In::frag_t lds_frag(const char* tile, int base, int jb, int ks) {
  using G = Geo<D, In::kES>;
  const char* row = tile + jb * 32 * G::kRowBytes;
  if constexpr (In::kES == 2) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(row + (base ^ (ks << 5)));
    return __builtin_bit_cast(typename In::frag_t, v);
  } else {
    const int o = base ^ (ks << 6);
    const f32x4 lo = *reinterpret_cast<const f32x4*>(row + o);
    const f32x4 hi = *reinterpret_cast<const f32x4*>(row + (o ^ 16));
    return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// fp16 image of a staged student tile (backward, bf16 inputs), laid out for the transposed
// gradient reads: D / 32 blocks of 32 columns, each [kBC rows][64 bytes], blocks kBlkBytes
// apart; in row r the two 32-byte halves of a block swap when bit 1 of r is set.  A
// transposed read (per 16-lane group four consecutive rows, 32 bytes each; 512 bytes in all)
// touches every bank once per 32 lanes, and its rows, halves and block are immediates on one
// per-lane base.  The 64 bytes between blocks put the 16 chunks of one row, which a group of
// 16 lanes converts together, on distinct banks.
template <int D>
struct ImgGeo {
  static constexpr int kBlkBytes = kBC * 64 + 64;
  static constexpr int kBytes = (D / 32) * kBlkBytes;
  // byte offset of chunk c (columns 8 c .. 8 c + 7) of row r
  __device__ static __forceinline__ int off(int r, int c) {
    return (c >> 2) * kBlkBytes + r * 64 + ((((c >> 1) ^ (r >> 1)) & 1) << 5) + ((c & 1) << 4);
  }
  // per-lane base of the transposed reads: lane s of 16-lane group g addresses row
  // 4 hh + s / 4 of an 8-row group, columns 16 (g % 2) + 4 (s % 4) .. +3 of the block
  __device__ static __forceinline__ int trb_base(int lane) {
    const int s = lane & 15, g = lane >> 4, hh = lane >> 5;
    const int r = 4 * hh + (s >> 2);
    return r * 64 + ((((g & 1) ^ (r >> 1)) & 1) << 5) + 8 * (s & 3);
  }
};

// ------------------------------------------------------------------ LDS read pipelines
// A single wave only sustains about 30 B/clk of LDS reads with a few reads in flight, while
// its MFMAs consume a 1 KB fragment per 32 cycles; so matrix phases request fragments far
// ahead of their MFMAs: before each MFMA, further fragments are requested while at most
// MAXOPS reads are outstanding (the LGKM counter tracks 15).  Measured best at 32 heads x
// 32K: 10 in the forward (1% faster than 8, 11 or 12, which the registers of its current
// pipeline only just hold) and 6 in the backward, whose phases hold more registers (7 and 8 no
// better; 12 was 2% slower).
constexpr int kFwdLdsOps = 10;
constexpr int kBwdLdsOps = 6;

template <int NG, int NF, int OPS_G, int OPS_S, int MAXOPS>
struct LoadSchedule {
  // LDS instructions of fragment k: OPS_G per gradient fragment, OPS_S per score fragment
  static constexpr int ops(int k) { return k < NG ? OPS_G : OPS_S; }
  // upto[f]: fragments [0, upto[f]) are requested before the MFMA of fragment f.  The
  // fragment an MFMA consumes is always requested before it, even when its reads alone
  // exceed MAXOPS (an fp32 gradient fragment takes 8).
  static constexpr std::array<int, NF> make() {
    std::array<int, NF> a{};
    int issued = 0;
    for (int f = 0; f < NF; ++f) {
      int inflight = 0;
      for (int k = f; k < issued; ++k) inflight += ops(k);
      while (issued < NF && inflight + ops(issued) <= MAXOPS) inflight += ops(issued++);
      if (issued < f + 1) issued = f + 1;
      a[f] = issued;
    }
    return a;
  }
  static constexpr std::array<int, NF> upto = make();
  static constexpr bool covers() {
    for (int f = 0; f < NF; ++f)
      if (upto[f] < f + 1) return false;
    return true;
  }
  static_assert(covers(), "every MFMA's fragment is requested before it");
};

// ------------------------------------------------------------------ forward
// Online update of one lane's row statistics with the 16 columns it holds of a 32x32
// score block (raw scores S; logits z = scale S; c2 = scale log2 e).
//   b: exponent bias in use (fp32), the sums are taken as exp2(S c2 + b);
//   l: sum of exp2(S c2 + b);  acc_a: sum of exp2(S_t c2 + b_t) (S_t - S_s).
// The bias is carried as the exact fp32 value that entered every exponent, so the
// rescale factors (exp2(b_new - b_old)) and the final LSE / KL use exactly the offsets
// the sums were taken with.  A block keeps the bias in use unless its largest exponent
// would exceed 2^32; then the bias moves to the block's maximum.  Masked columns contribute
// exactly zero (the select is on the exponential itself).  REL: the relation, whose
// diagonal entry j == i is left out of the sums (the kernel adds it exactly at the end).
template <bool MASK, bool CAUSAL, bool REL>
__device__ __forceinline__ void online_update(const f32x16& st, const f32x16& ss, int jb0, int i,
                                              int hh, int N, float c2, float& b_t, float& l_t,
                                              float& acc_a, float& b_s, float& l_s) {
  bool keep[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int j = jb0 + 8 * (r >> 2) + 4 * hh + (r & 3);
    keep[r] = !MASK || ((j < N) && (!CAUSAL || j <= i) && (!REL || j != i));
  }
  float mx_t = kNegBig, mx_s = kNegBig;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    mx_t = fmaxf(mx_t, keep[r] ? st[r] : kNegBig);
    mx_s = fmaxf(mx_s, keep[r] ? ss[r] : kNegBig);
  }
  const float bn_t = fmaf(mx_t, c2, b_t) > 32.f ? -mx_t * c2 : b_t;
  const float bn_s = fmaf(mx_s, c2, b_s) > 32.f ? -mx_s * c2 : b_s;
  const float alpha_t = fast_exp2(bn_t - b_t);
  const float alpha_s = fast_exp2(bn_s - b_s);
  float e_t[16], e_s[16], dd[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float et = fast_exp2(fmaf(st[r], c2, bn_t));
    const float es = fast_exp2(fmaf(ss[r], c2, bn_s));
    e_t[r] = keep[r] ? et : 0.f;
    e_s[r] = keep[r] ? es : 0.f;
    dd[r] = keep[r] ? et * (st[r] - ss[r]) : 0.f;
  }
  // pairwise sums of the 16 terms
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) {
#pragma unroll
    for (int r = 0; r < s; ++r) {
      e_t[r] += e_t[r + s];
      e_s[r] += e_s[r + s];
      dd[r] += dd[r + s];
    }
  }
  l_t = fmaf(l_t, alpha_t, e_t[0]);
  acc_a = fmaf(acc_a, alpha_t, dd[0]);
  l_s = fmaf(l_s, alpha_s, e_s[0]);
  b_t = bn_t;
  b_s = bn_s;
}

// Fast path of the online update for a block without masked entries: the exponentials use
// the lane's current biases as they are, so no block maximum is formed.  The block is
// accumulated only if both block sums are at most 2^64, which bounds every exponential
// (and rules out inf / NaN); then the running sums stay finite and exact in the sense of
// the bias form above.  Otherwise (a row's first block when the bias is still the
// empty-row value of the cross relation, or a row maximum that grew by more than 64 in log2
// units over the bias) nothing is changed and the caller runs the exact path.  Returns
// whether the block was accumulated.
__device__ __forceinline__ bool online_update_fast(const f32x16& st, const f32x16& ss, float c2,
                                                   float b_t, float b_s, float& l_t,
                                                   float& acc_a, float& l_s) {
  float lt0 = 0.f, lt1 = 0.f, ls0 = 0.f, ls1 = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float et0 = fast_exp2(fmaf(st[r], c2, b_t));
    const float es0 = fast_exp2(fmaf(ss[r], c2, b_s));
    const float et1 = fast_exp2(fmaf(st[r + 1], c2, b_t));
    const float es1 = fast_exp2(fmaf(ss[r + 1], c2, b_s));
    lt0 += et0;
    ls0 += es0;
    a0 = fmaf(et0, st[r] - ss[r], a0);
    lt1 += et1;
    ls1 += es1;
    a1 = fmaf(et1, st[r + 1] - ss[r + 1], a1);
  }
  const float sum_t = lt0 + lt1, sum_s = ls0 + ls1;
  const bool ok = sum_t <= 0x1p64f && sum_s <= 0x1p64f;
  if (ok) {
    l_t += sum_t;
    l_s += sum_s;
    acc_a += a0 + a1;
  }
  return ok;
}

__device__ __forceinline__ u32x4 bf16x8_to_f16x8_bits(const bf16x8& v) {
  const u32x4 w = __builtin_bit_cast(u32x4, v);
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float lo = __uint_as_float(w[q] << 16);
    const float hi = __uint_as_float(w[q] & 0xffff0000u);
    // exact for values representable in fp16; round-toward-zero only matters beyond that
    o[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
  return o;
}

// Score contraction of one 32 x 32 block of the forward as a software pipeline: the LDS
// reads of the key fragments run ahead of their MFMAs with at most kFwdLdsOps reads in
// flight.  After MFMA I the callback extra(I) places independent vector work (the previous
// block's exponentials) in the same scheduling region as the reads for the next MFMA, so a
// wave keeps its vector unit busy while its own MFMAs run.
template <class In, int D, class Extra>
__device__ __forceinline__ void score_pipeline(const char* tile_t, const char* tile_s, int fbase,
                                               int jb, const typename In::frag_t (&qt)[D / 16],
                                               const typename In::frag_t (&qs)[D / 16],
                                               f32x16& st, f32x16& ss, Extra&& extra) {
  using frag_t = typename In::frag_t;
  constexpr int KS = D / 16, NF = 2 * KS;
  using S = LoadSchedule<0, NF, 1, In::kES == 2 ? 1 : 2, kFwdLdsOps>;
  frag_t fr[NF];
  auto load = [&](auto fc) __attribute__((always_inline)) {
    constexpr int f = decltype(fc)::value, ks = f / 2, m = f % 2;
    fr[f] = lds_frag<In, D>(m ? tile_s : tile_t, fbase, jb, ks);
  };
  auto mma = [&](auto fc) __attribute__((always_inline)) {
    constexpr int f = decltype(fc)::value, ks = f / 2, m = f % 2;
    if constexpr (m == 0) st = mma_k16(fr[f], qt[ks], st);
    else ss = mma_k16(fr[f], qs[ks], ss);
  };
  st = f32x16{};
  ss = f32x16{};
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((
      [&] {
        constexpr int lo = I == 0 ? 0 : S::upto[I == 0 ? 0 : I - 1];
        [&]<int... J>(std::integer_sequence<int, J...>) {
          (load(std::integral_constant<int, lo + J>{}), ...);
        }(std::make_integer_sequence<int, S::upto[I] - lo>{});
        __builtin_amdgcn_sched_barrier(0);
        mma(std::integral_constant<int, I>{});
        __builtin_amdgcn_sched_barrier(0);
        extra(std::integral_constant<int, I>{});
      }()), ...);
  }(std::make_integer_sequence<int, NF>{});
  __builtin_amdgcn_sched_barrier(0);
}

// Sum of squares of this lane's part of its row (8 elements per fragment), in fp64: the
// products of bf16 or fp32 values are exact there, and so is, up to 2^-53, their sum.
template <class In, int D>
__device__ __forceinline__ double row_sq_sum(const typename In::frag_t (&q)[D / 16]) {
  double acc = 0.0;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if constexpr (In::kES == 2) {
      const u32x4 w = __builtin_bit_cast(u32x4, q[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double lo = (double)__uint_as_float(w[e] << 16);
        const double hi = (double)__uint_as_float(w[e] & 0xffff0000u);
        acc = fma(lo, lo, acc);
        acc = fma(hi, hi, acc);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fma((double)q[ks][e], (double)q[ks][e], acc);
    }
  }
  return acc;
}

// REL: the relation softmax(scale X X^T); its diagonal score S_ii = |X_i|^2 is the row's
// reference (below).  !REL: the cross relation softmax(scale A B^T), no reference entry.
template <class In, int D, bool CAUSAL, bool REL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void relkl_fwd_kernel(const FwdLaunch L) {
  using elem_t = typename In::elem_t;
  using frag_t = typename In::frag_t;
  using G = Geo<D, In::kES>;
  constexpr int KS = D / 16;  // 16-deep steps over d
  constexpr int kStage = 2 * G::kTileBytes;

  // two stage buffers: a step reads one while its copies fill the other
  __shared__ __attribute__((aligned(1024))) char lds0[kStage];
  __shared__ __attribute__((aligned(1024))) char lds1[kStage];
  __shared__ double red[kWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;

  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int mi = member_of(L, g);
  const FwdArgs& a = L.m[mi];
  const int N = a.N;
  const int w = g - member_begin(L, mi);
  const int unit = w / a.row_tiles;
  const int it = w - unit * a.row_tiles;
  const int I = CAUSAL ? (a.row_tiles - 1 - it) : it;  // longest causal rows first
  const int b = unit / a.H, h = unit - (unit / a.H) * a.H;
  const int hin = head_of(L, a.map_off, h);
  const elem_t* xt = reinterpret_cast<const elem_t*>(a.x_t) + b * a.t_sb + hin * a.t_sh;
  const elem_t* xs = reinterpret_cast<const elem_t*>(a.x_s) + b * a.s_sb + hin * a.s_sh;
  // key-side rows: the same matrix for the relation, B for the cross relation (same layout)
  const int64_t yo_t = b * a.t_sb + hin * a.t_sh, yo_s = b * a.s_sb + hin * a.s_sh;
  const char* xt_c = reinterpret_cast<const char*>(
      a.y_t ? reinterpret_cast<const elem_t*>(a.y_t) + yo_t : xt);
  const char* xs_c = reinterpret_cast<const char*>(
      a.y_s ? reinterpret_cast<const elem_t*>(a.y_s) + yo_s : xs);
  const int64_t tsn_b = a.t_sn * In::kES, ssn_b = a.s_sn * In::kES;

  const int i0 = I * kBR;
  const int ib0 = i0 + 32 * wave;  // first row of this wave
  const int row = ib0 + l32;       // this lane's row

  const int j_end = CAUSAL ? min(N, i0 + kBR) : N;
  const int n_tiles = (j_end + kBC - 1) / kBC;
  dma_tile<D, In::kES>(xt_c, tsn_b, 0, N, lds0, wave, lane);
  dma_tile<D, In::kES>(xs_c, ssn_b, 0, N, lds0 + G::kTileBytes, wave, lane);

  // Own rows as B operands: lane (l32, hh) holds elements 16 ks + 8 hh .. +7 of its row.
  frag_t qt[KS], qs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (row < N) {
      qt[ks] = load_frag_global<In>(xt + (int64_t)row * a.t_sn + 16 * ks + 8 * hh);
      qs[ks] = load_frag_global<In>(xs + (int64_t)row * a.s_sn + 16 * ks + 8 * hh);
    } else {
      qt[ks] = frag_t{};
      qs[ks] = frag_t{};
    }
  }

  const int fbase = frag_base<In, D>(l32, hh);
  const float c2 = a.c2;
  const float b_init = -kNegBig * c2;  // bias of an empty row: every real bias is below it
  float b_t = b_init, l_t = 0.f, acc_a = 0.f, b_s = b_init, l_s = 0.f;
  // The relation's diagonal entry carries most of a row's mass (S_ii = |X_i|^2 against
  // off-diagonal scores of about |X|), so in fp32 its own rounding would dominate the KL
  // of nearly equal teacher and student rows.  It is therefore left out of the sweep and
  // added exactly at the end, from S_ii in fp64 (the two half-waves holding the row each
  // sum their half).  The row's bias starts at -c2 S_ii, which makes the diagonal's own
  // exponential 2^rho with rho the (tiny) rounding residual of that bias.
  double sq_t = 0.0, sq_s = 0.0;
  if constexpr (REL) {
    sq_t = row_sq_sum<In, D>(qt);
    sq_s = row_sq_sum<In, D>(qs);
    sq_t += __shfl_xor(sq_t, 32);
    sq_s += __shfl_xor(sq_s, 32);
    b_t = (float)(-(double)c2 * sq_t);
    b_s = (float)(-(double)c2 * sq_s);
  }

  // Software pipeline over 32-key blocks, which alternate between two score buffers: the
  // exponentials and sums of a block without masked entries run inside the MFMA sequence of
  // the next block (one element of the 16 per MFMA at d = 128), with both at the raised
  // issue priority.  The order of every sum is that of online_update_fast.  A block with
  // masked entries (the diagonal block of the relation, the causal diagonal block, the
  // ragged end) and the exact fallback run on their own.
  f32x16 stA = f32x16{}, ssA = f32x16{}, stB = f32x16{}, ssB = f32x16{};
  bool have_p = false, p_mask = false;  // a pending block, whether it has masked entries
  int p_jb0 = 0, p_par = 0;             // its first column, its buffer (A: 0, B: 1)
  auto finish = [&](const f32x16& pt, const f32x16& ps) __attribute__((always_inline)) {
    if (p_mask)
      online_update<true, CAUSAL, REL>(pt, ps, p_jb0, row, hh, N, c2, b_t, l_t, acc_a, b_s, l_s);
    else if (!online_update_fast(pt, ps, c2, b_t, b_s, l_t, acc_a, l_s))
      online_update<false, CAUSAL, REL>(pt, ps, p_jb0, row, hh, N, c2, b_t, l_t, acc_a, b_s, l_s);
  };
  // Block jb of the tile: scores into (st, ss) while the pending block (pt, ps) is reduced.
  auto block = [&](auto jbc, int kt, const char* tile_t, const char* tile_s, f32x16& st,
                   f32x16& ss, const f32x16& pt, const f32x16& ps) __attribute__((always_inline)) {
    constexpr int jb = decltype(jbc)::value;
    const int jb0 = kt * kBC + 32 * jb;
    if (jb0 >= N) return false;
    if (CAUSAL && jb0 > ib0 + 31) return false;  // above every row of the wave
    const bool need_mask = (CAUSAL && jb0 + 31 > ib0) || (jb0 + 32 > N) || (REL && jb0 == ib0);
    if (have_p && !p_mask) {
      constexpr int NF = 2 * KS, E = (16 + NF - 1) / NF;  // elements per MFMA slot
      float lt[2] = {0.f, 0.f}, ls[2] = {0.f, 0.f}, aa[2] = {0.f, 0.f};
      const float bt = b_t, bs = b_s;
      __builtin_amdgcn_s_setprio(1);
      // Element r's exponent arguments and exponentials go into one MFMA slot and its sums
      // into the next, so that no slot waits on an exponential it has just issued; the sums
      // keep their order, so the result is the same bit for bit.
      float ut[16], us[16], xt[16], xs[16];
      auto pre = [&](int r) __attribute__((always_inline)) {
        ut[r] = fmaf(pt[r], c2, bt);
        us[r] = fmaf(ps[r], c2, bs);
      };
      auto ex = [&](int r) __attribute__((always_inline)) {
        xt[r] = fast_exp2(ut[r]);
        xs[r] = fast_exp2(us[r]);
      };
      auto add = [&](int r) __attribute__((always_inline)) {
        if (r < 2) {  // an exponential is never -0, so this equals 0 + the exponential bitwise
          lt[r] = xt[r];
          ls[r] = xs[r];
        } else {
          lt[r & 1] += xt[r];
          ls[r & 1] += xs[r];
        }
        aa[r & 1] = fmaf(xt[r], pt[r] - ps[r], aa[r & 1]);
      };
      score_pipeline<In, D>(tile_t, tile_s, fbase, jb, qt, qs, st, ss,
                            [&](auto ic) __attribute__((always_inline)) {
        constexpr int I = decltype(ic)::value;
        constexpr int lo = I * E < 16 ? I * E : 16, hi = (I + 1) * E < 16 ? (I + 1) * E : 16;
#pragma unroll
        for (int r = lo; r < hi; ++r) pre(r);
#pragma unroll
        for (int r = lo; r < hi; ++r) ex(r);
#pragma unroll
        for (int r = (lo >= E ? lo - E : 0); r < (lo >= E ? lo : 0); ++r) add(r);
      });
#pragma unroll
      for (int r = 16 - E; r < 16; ++r) add(r);
      __builtin_amdgcn_s_setprio(0);
      const float sum_t = lt[0] + lt[1], sum_s = ls[0] + ls[1], sum_a = aa[0] + aa[1];
      const bool ok = sum_t <= 0x1p64f && sum_s <= 0x1p64f;
      // selects, not a branch, so that the KL products stay inside the MFMA sequence
      l_t = ok ? l_t + sum_t : l_t;
      l_s = ok ? l_s + sum_s : l_s;
      acc_a = ok ? acc_a + sum_a : acc_a;
      if (!ok)
        online_update<false, CAUSAL, REL>(pt, ps, p_jb0, row, hh, N, c2, b_t, l_t, acc_a, b_s, l_s);
    } else {
      if (have_p) finish(pt, ps);
      // the LDS-bound matrix part issues ahead of the partner wave's vector work
      __builtin_amdgcn_s_setprio(1);
      score_pipeline<In, D>(tile_t, tile_s, fbase, jb, qt, qs, st, ss, [](auto) {});
      __builtin_amdgcn_s_setprio(0);
    }
    have_p = true;
    p_mask = need_mask;
    p_jb0 = jb0;
    p_par = jb;
    return true;
  };
  static_assert(kBC == 64, "two 32-key blocks per tile, one per score buffer");
  auto step = [&](int kt, const char* cur, char* nxt) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (kt + 1 < n_tiles) {
      dma_tile<D, In::kES>(xt_c, tsn_b, (kt + 1) * kBC, N, nxt, wave, lane);
      dma_tile<D, In::kES>(xs_c, ssn_b, (kt + 1) * kBC, N, nxt + G::kTileBytes, wave, lane);
    }
    const char* tile_t = cur;
    const char* tile_s = cur + G::kTileBytes;
    // blocks are consecutive, so the pending block of block 0 is in B and that of block 1 in A
    if (block(std::integral_constant<int, 0>{}, kt, tile_t, tile_s, stA, ssA, stB, ssB))
      block(std::integral_constant<int, 1>{}, kt, tile_t, tile_s, stB, ssB, stA, ssA);
  };
  for (int kt = 0; kt < n_tiles; kt += 2) {
    step(kt, lds0, lds1);
    if (kt + 1 < n_tiles) step(kt + 1, lds1, lds0);
  }
  if (have_p) {
    if (p_par == 0) finish(stA, ssA);
    else finish(stB, ssB);
  }

  // Merge the two half-waves (lanes l and l ^ 32 hold the same row) onto one bias.
  const float ob_t = __shfl_xor(b_t, 32), ol_t = __shfl_xor(l_t, 32);
  const float oa = __shfl_xor(acc_a, 32);
  const float ob_s = __shfl_xor(b_s, 32), ol_s = __shfl_xor(l_s, 32);
  const float B_t = fminf(b_t, ob_t), B_s = fminf(b_s, ob_s);
  const float f1t = fast_exp2(B_t - b_t), f2t = fast_exp2(B_t - ob_t);
  const float f1s = fast_exp2(B_s - b_s), f2s = fast_exp2(B_s - ob_s);
  const float L_t = l_t * f1t + ol_t * f2t;
  const float A_t = acc_a * f1t + oa * f2t;
  const float L_s = l_s * f1s + ol_s * f2s;
  // Finish the row, in log2 units: with every term exp2(S c2 + B),
  //   LSE = ln2 (log2 L - B),
  //   KL  = ln2 (c2 A_t / L_t + (B_t - B_s) - log2(L_t / L_s))
  // (KL_i = E_t[z_t - z_s] - (LSE_t - LSE_s), with the LSE difference taken as a ratio).
  float kl, lse_t, lse_s, dd = 0.f;
  if constexpr (REL) {
    // The sums hold the off-diagonal terms (L', A'); the diagonal's own term is 2^rho with
    // rho = c2 S_ii + B, exact in fp64.  With lambda = L' 2^-rho and D = S_t,ii - S_s,ii:
    //   KL  = scale (A'_t - D L'_t) / L_t - log1p((lambda_t - lambda_s) / (1 + lambda_s)),
    //   LSE = scale S_ii + log1p(lambda),
    //   R_s(i,i) - R_t(i,i) = 1 / (1 + lambda_s) - 1 / (1 + lambda_t),
    // in which the large diagonal terms have cancelled exactly, so that a row whose KL is
    // tiny against its LSE keeps relative precision, and a row with no off-diagonal entry
    // gives KL = 0 and R(i,i) = 1 exactly.  When the bias had to move far below the
    // diagonal's (a row dominated by other entries, rho < -30) the plain form is used with
    // the diagonal's term added to the sums.
    const double rho_t = (double)c2 * sq_t + (double)B_t;
    const double rho_s = (double)c2 * sq_s + (double)B_s;
    const float dg = (float)(sq_t - sq_s);  // D = S_t,ii - S_s,ii
    const float e_t = fast_exp2((float)rho_t), e_s = fast_exp2((float)rho_s);
    if (rho_t >= -30.0 && rho_s >= -30.0) {
      const float lam_t = L_t / e_t, lam_s = L_s / e_s;
      kl = a.scale * ((A_t - dg * L_t) / (e_t + L_t)) - log1pf((lam_t - lam_s) / (1.f + lam_s));
      dd = (lam_t - lam_s) / ((1.f + lam_s) * (1.f + lam_t));
      lse_t = (float)((double)a.scale * sq_t + (double)log1pf(lam_t));
      lse_s = (float)((double)a.scale * sq_s + (double)log1pf(lam_s));
    } else {
      const float Lt = e_t + L_t, Ls = e_s + L_s, At = fmaf(e_t, dg, A_t);
      kl = kLn2 * (c2 * (At / Lt) + (B_t - B_s) - log2f(Lt / Ls));
      dd = e_s / Ls - e_t / Lt;
      lse_t = (log2f(Lt) - B_t) * kLn2;
      lse_s = (log2f(Ls) - B_s) * kLn2;
    }
  } else {
    kl = kLn2 * (c2 * (A_t / L_t) + (B_t - B_s) - log2f(L_t / L_s));
    lse_t = (log2f(L_t) - B_t) * kLn2;
    lse_s = (log2f(L_s) - B_s) * kLn2;
  }
  double kl_sum = 0.0;
  if (hh == 0 && row < N) {
    const int64_t o = (int64_t)unit * N + row;
    a.lse_t[o] = lse_t;
    a.lse_s[o] = lse_s;
    if (a.row_kl) a.row_kl[o] = kl;
    if (REL && a.diag_delta) a.diag_delta[o] = dd;
    kl_sum = (double)kl;
  }
  // Deterministic workgroup sum in fp64.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kl_sum += __shfl_xor(kl_sum, off);
  if (lane == 0) red[wave] = kl_sum;
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) s += red[q];
    a.partial[w] = s;
  }
}

// Fixed-order fp64 reduction of the per-workgroup partial sums into the fp32 loss: block 0
// sums every member's partials into the total, block k >= 1 member k-1's into its own
// loss (when requested).
__global__ __launch_bounds__(256) void loss_reduce_kernel(const LossOut o) {
  __shared__ double red[256];
  const int blk = blockIdx.x;
  float* out = blk == 0 ? o.total : o.member[blk - 1];
  if (out == nullptr) return;
  const int lo = blk == 0 ? 0 : o.begin[blk - 1];
  const int hi = blk == 0 ? o.begin[o.n] : o.begin[blk];
  double s = 0.0;
  for (int k = lo + (int)threadIdx.x; k < hi; k += 256) s += o.partial[k];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off >= 1; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = (float)red[0];
}

// ------------------------------------------------------------------ backward
// W block (times 2^14) of one lane: the 16 columns j = jb0 + 8 (r/4) + 4 hh + (r%4) of
// its row i, from the transposed score blocks st / ss (raw scores) and the log2 row
// statistics r (R * 2^14 = exp2(S c2 - r)).
//   row term  (entry (i, j) of dZ, normalised by the statistic of row i):  kept if j <= i
//   col term  (entry (j, i) of dZ, normalised by the statistic of row j):  kept if i <= j
// ROW / COL: which terms the block takes (the symmetric relation: both where the mask keeps
// them -- the row term below the diagonal, the column term above, both on the diagonal
// block; the cross relation's dA pass only row terms, its dB pass only column terms);
// DIAG: the causal diagonal block, masked per element; TAIL zeroes columns j >= N (their
// staged rows and statistics are copies of row N-1); SUB: the block holds the relation's
// diagonal entry (i, i), which takes wd2 = 2 (R_s(i,i) - R_t(i,i)) 2^14 as given by the
// forward (row and column term) instead of the recomputed difference: with R(i,i) near 1
// the fp32 statistics cannot resolve it.
template <bool ROW, bool COL, bool DIAG, bool TAIL, bool SUB = false>
__device__ __forceinline__ void make_w(const f32x16& st, const f32x16& ss, float rt, float rs,
                                       const float* clt, const float* cls, int hh, int di,
                                       int n_left, float c2, float wd2, f32x8 (&w32)[2]) {
  float wv[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 ct4 = f32x4{0.f, 0.f, 0.f, 0.f}, cs4 = ct4;
    if constexpr (COL) {
      ct4 = *reinterpret_cast<const f32x4*>(clt + 8 * q + 4 * hh);
      cs4 = *reinterpret_cast<const f32x4*>(cls + 8 * q + 4 * hh);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = 4 * q + t;
      const int dj = 8 * q + 4 * hh + t;  // j - jb0
      float v = 0.f;
      if constexpr (ROW) {
        const float rt_ = fast_exp2(fmaf(ss[r], c2, -rs)) - fast_exp2(fmaf(st[r], c2, -rt));
        v = DIAG ? (dj <= di ? rt_ : 0.f) : rt_;
      }
      if constexpr (COL) {
        const float ct_ = fast_exp2(fmaf(ss[r], c2, -cs4[t])) - fast_exp2(fmaf(st[r], c2, -ct4[t]));
        const float cm = DIAG ? (dj >= di ? ct_ : 0.f) : ct_;
        // a difference of two exponentials is never -0, so v = cm equals 0 + cm bitwise
        if constexpr (ROW) v += cm;
        else v = cm;
      }
      if constexpr (SUB) v = dj == di ? wd2 : v;
      if constexpr (TAIL) v = dj < n_left ? v : 0.f;
      wv[r] = v;
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) w32[kb][e] = wv[8 * kb + e];
}

template <class Op>
__device__ __forceinline__ typename Op::gfrag_t w_frag(const f32x8& w) {
  if constexpr (Op::kES == 2) {
    return __builtin_convertvector(w, f16x8);  // round to nearest even, two per instruction
  } else {
    return w;
  }
}

// Gradient-contraction B fragment: X_s[j][d] for d = 32 mb + l32 and the 8 k-slots
// j = jbase + 8 (e/4) + 4 hh + (e%4) (jbase = 32 jb + 16 kb), read transposed from the
// row-major key tile.  ds_read_b64_tr_b16: in each 16-lane group, lane s gives the
// address of row (r0 + s/4), columns c0 + 4 (s%4) .. +3, and lane q receives column
// c0 + q of rows r0 .. r0 + 3.  Here r0 = jbase + 8 half + 4 hh and c0 = 32 mb + 16 (g%2)
// for lane group g.  In the swizzled key tile (fp16 reserve copies of the cross relation)
// the row swizzle does not depend on jb or kb (multiples of 16 rows), and mb only flips chunk
// bits 2-3, so the address is a per-lane base for each half, XOR (mb << 6), plus the
// immediate jbase rows; in the fp16 image of bf16 inputs (ImgGeo) the whole offset past one
// per-lane base is an immediate.
template <int D>
__device__ __forceinline__ int trb_base(int lane, int half) {
  using G = Geo<D, 2>;
  const int s = lane & 15, g = lane >> 4, hh = lane >> 5;
  const int r = 8 * half + 4 * hh + (s >> 2);
  const int col = 16 * (g & 1) + 4 * (s & 3);
  return G::off(r, col >> 3) + (col & 7) * 2;
}

template <class Op, int D>
__device__ __forceinline__ typename Op::gfrag_t grad_bfrag(const char* tile, int jbase, int mb,
                                                           int lane, int tb0, int tb1) {
  using G = Geo<D, Op::kES>;
  if constexpr (Op::kConvert) {  // the fp16 image (ImgGeo); tb0 from ImgGeo::trb_base
    const char* p = tile + tb0 + (mb * ImgGeo<D>::kBlkBytes + jbase * 64);
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p);
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 8 * 64));
    const u32x2 a0 = __builtin_bit_cast(u32x2, v0), a1 = __builtin_bit_cast(u32x2, v1);
    return __builtin_bit_cast(f16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
  } else if constexpr (Op::kES == 2) {
    const char* rows = tile + jbase * G::kRowBytes;
    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(rows + (tb0 ^ (mb << 6))));
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(rows + (tb1 ^ (mb << 6))));
    const u32x2 a0 = __builtin_bit_cast(u32x2, v0), a1 = __builtin_bit_cast(u32x2, v1);
    return __builtin_bit_cast(f16x8, u32x4{a0[0], a0[1], a1[0], a1[1]});
  } else {
    const int d = 32 * mb + (lane & 31), hh = lane >> 5;
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = jbase + 8 * (e >> 2) + 4 * hh + (e & 3);
      f[e] = *reinterpret_cast<const float*>(tile + G::off(r, d >> 2) + (d & 3) * 4);
    }
    return f;
  }
}

// Matrix phase of the backward as an explicit software pipeline over "fragments": first the
// 2 MB gradient B fragments of the previous block (two transposed 8-byte LDS reads each),
// then the 2 KS score A fragments of the current block (one 16-byte read each), one MFMA
// per fragment, with the reads running ahead of their MFMAs as LoadSchedule allows.
// Scheduling barriers keep that order; consecutive MFMAs use different accumulators.

// Gradient fragment f of a matrix phase: k-half h = f / MB, output block mb = f % MB.
template <class Op, int D, int F>
__device__ __forceinline__ typename Op::gfrag_t grad_frag(const char* gtile, int jbg, int lane,
                                                          int tb0, int tb1) {
  constexpr int MB = D / 32, mb = F % MB, h = F / MB;
  return grad_bfrag<Op, D>(gtile, jbg + 16 * h, mb, lane, tb0, tb1);
}

template <class Op, int D>
__device__ __forceinline__ void m_pipeline(const char* gtile, int jbg, const char* stile, int jbs,
                                           int fbase, int lane, int tb0, int tb1,
                                           const typename Op::gfrag_t& wf0,
                                           const typename Op::gfrag_t& wf1,
                                           const typename Op::frag_t (&qt)[D / 16],
                                           const typename Op::frag_t (&qs)[D / 16],
                                           f32x16 (&acc)[D / 32], f32x16& st, f32x16& ss) {
  using G = Geo<D, Op::kES>;
  constexpr int KS = D / 16, MB = D / 32;
  constexpr int NG = 2 * MB;
  constexpr int NF = NG + 2 * KS;
  using S = LoadSchedule<NG, NF, Op::kES == 2 ? 2 : 8, Op::kES == 2 ? 1 : 2, kBwdLdsOps>;
  typename Op::gfrag_t gr[NG];
  typename Op::frag_t sr[2 * KS];
  auto load = [&](auto fc) __attribute__((always_inline)) {
    constexpr int f = decltype(fc)::value;
    if constexpr (f < NG) {
      gr[f] = grad_frag<Op, D, f>(gtile, jbg, lane, tb0, tb1);
    } else {
      constexpr int k = f - NG, ks = k / 2, m = k % 2;
      sr[k] = lds_frag<Op, D>(m ? stile + G::kTileBytes : stile, fbase, jbs, ks);
    }
  };
  auto mma = [&](auto fc) __attribute__((always_inline)) {
    constexpr int f = decltype(fc)::value;
    if constexpr (f < NG) {
      constexpr int mb = f % MB, h = f / MB;
      acc[mb] = mma_k16(h ? wf1 : wf0, gr[f], acc[mb]);
    } else {
      constexpr int k = f - NG, ks = k / 2, m = k % 2;
      if constexpr (m == 0) st = mma_k16(sr[k], qt[ks], st);
      else ss = mma_k16(sr[k], qs[ks], ss);
    }
  };
  st = f32x16{};
  ss = f32x16{};
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((
      [&] {
        constexpr int lo = I == 0 ? 0 : S::upto[I == 0 ? 0 : I - 1];
        [&]<int... J>(std::integer_sequence<int, J...>) {
          (load(std::integral_constant<int, lo + J>{}), ...);
        }(std::make_integer_sequence<int, S::upto[I] - lo>{});
        __builtin_amdgcn_sched_barrier(0);
        mma(std::integral_constant<int, I>{});
        __builtin_amdgcn_sched_barrier(0);
      }()), ...);
  }(std::make_integer_sequence<int, NF>{});
}

// Backward work decomposition: a workgroup of 8 waves (two per SIMD) owns 256 rows, 32 per
// wave, and sweeps the whole key range in key tiles of 64 rows (two 32-key blocks).  fp32
// operands take twice the registers: there a workgroup is 4 waves (one per SIMD, which may
// then hold 512 registers) owning 128 rows, and nothing runs beside a wave's phases.
// MODE 0 is the relation gradient (own rows and staged rows are the same matrix: row and
// column terms).  The cross relation softmax(A B^T) takes two passes: MODE 1 owns rows of
// A and stages rows of B (row terms only: dA = scale dZ B_s, keys j <= i when causal);
// MODE 2 owns rows of B and stages rows of A with their statistics (column terms only:
// dB = scale dZ^T A_s, queries i >= j when causal).
// For each block n a wave runs
//    M(n): gradient MFMAs of block n-1 (W(n-1) X_s) and score MFMAs of block n
//    V(n): W(n) from the scores of block n (exp / VALU work)
// The waves drift freely between the barriers that separate key tiles, so one wave's
// vector work overlaps its SIMD partner's matrix work.
// Bf16Op (bf16 inputs, MODE 0) reads the caller's bf16 rows: the scores contract them as
// they are (as the forward does), and every staged student tile also gets an IEEE fp16
// image in LDS (exact for 2^-17 <= |x| < 65504), which the gradient contraction reads with W
// carried as fp16: each wave converts the 16-byte chunks it copied itself, after its own
// copies have landed and before the barrier that publishes the tile, into the column-blocked
// layout of ImgGeo (one address addition per matrix phase for all of its transposed reads).
template <class Op, int D, bool CAUSAL, bool OUT_F32, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(bwd_waves(Op::kES == 4) * kWave,
                                                      bwd_waves(Op::kES == 4) * kWave),
                          amdgpu_waves_per_eu(bwd_waves(Op::kES == 4) / 4,
                                              bwd_waves(Op::kES == 4) / 4)))
void relkl_bwd_kernel(const BwdLaunch L) {
  using elem_t = typename Op::elem_t;
  using frag_t = typename Op::frag_t;
  using gfrag_t = typename Op::gfrag_t;
  using G = Geo<D, Op::kES>;
  constexpr int KS = D / 16;
  constexpr int MB = D / 32;  // 32-wide output blocks over d
  using P = ImgGeo<D>;
  constexpr int kStats = 2 * kBC * 4;
  // stage layout: [teacher tile][student tile]([student fp16 image])[teacher stats][student stats]
  constexpr int kTileB = G::kTileBytes;
  constexpr int kImgB = Op::kConvert ? P::kBytes : 0;
  constexpr int kGradOff = Op::kConvert ? 2 * kTileB : kTileB;
  constexpr int kStatsOff = 2 * kTileB + kImgB;
  constexpr int kStage = kStatsOff + kStats;
  constexpr int kW = bwd_waves(Op::kES == 4);  // waves of the workgroup
  constexpr int kRowsWG = 32 * kW;               // rows it owns
  constexpr int kDma = kBC * G::kCPR / (kWave * kW);  // DMA instructions per wave per tile
  static_assert(kBC * G::kCPR % (kWave * kW) == 0, "tile must split evenly over the waves");
  static_assert(MODE == 0 || !Op::kConvert, "the cross relation reads fp16 images");

  // Stage buffers: three when they fit in the LDS, else two (fp32, d = 128).
  constexpr int kStages = 3 * kStage <= 160 * 1024 ? 3 : 2;
  __shared__ __attribute__((aligned(1024))) char lds[kStages * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;

  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const int mi = member_of(L, g);
  const BwdArgs& a = L.m[mi];
  const int N = a.N;
  const int w = g - member_begin(L, mi);
  const int split = w % a.splits;
  const int wt = w / a.splits;
  const int unit = wt / a.row_tiles;
  // the cross dA pass does more work for later row tiles under the causal mask: run those
  // first, as the forward does (the dB pass already starts with its longest row tiles)
  const int I = (CAUSAL && MODE == 1) ? a.row_tiles - 1 - (wt - unit * a.row_tiles)
                                      : wt - unit * a.row_tiles;
  const int b = unit / a.H, h = unit - (unit / a.H) * a.H;
  const int hin = head_of(L, a.map_off, h);

  // Operands: the caller's rows in place (through the head map and strides), or dense
  // [unit][N][D] copies from the reserve; own rows from x, staged key rows from y (the same
  // matrix for the relation).
  const elem_t* xt;
  const elem_t* xs;
  const elem_t* yt;
  const elem_t* ys;
  int64_t tsn, ssn;
  if (a.x_dense) {
    xt = reinterpret_cast<const elem_t*>(a.x_t) + (int64_t)unit * N * D;
    xs = reinterpret_cast<const elem_t*>(a.x_s) + (int64_t)unit * N * D;
    yt = reinterpret_cast<const elem_t*>(a.y_t) + (int64_t)unit * N * D;
    ys = reinterpret_cast<const elem_t*>(a.y_s) + (int64_t)unit * N * D;
    tsn = D;
    ssn = D;
  } else {
    xt = reinterpret_cast<const elem_t*>(a.x_t) + b * a.t_sb + hin * a.t_sh;
    xs = reinterpret_cast<const elem_t*>(a.x_s) + b * a.s_sb + hin * a.s_sh;
    yt = xt;
    ys = xs;
    tsn = a.t_sn;
    ssn = a.s_sn;
  }
  const char* yt_c = reinterpret_cast<const char*>(yt);
  const char* ys_c = reinterpret_cast<const char*>(ys);
  const int64_t tsn_b = tsn * Op::kES, ssn_b = ssn * Op::kES;
  // row strides in bytes are below 2^24 (checked on the host), so a clamped row (< 64)
  // times the stride plus a chunk offset is a 24-bit multiply-add
  const uint32_t tsn_u24 = (uint32_t)tsn_b, ssn_u24 = (uint32_t)ssn_b;
  // The forward's LSE vectors (nats); the kernel uses them as log2 statistics
  // r = LSE log2(e) - 14, for which R(i, j) 2^14 = exp2(S_ij c2 - r_i).
  const float* own_t = a.lse_t + (int64_t)unit * N;
  const float* own_s = a.lse_s + (int64_t)unit * N;
  const float* stg_t = a.lc_t + (int64_t)unit * N;
  const float* stg_s = a.lc_s + (int64_t)unit * N;
  constexpr float kLog2e = 1.4426950408889634f;

  const int i0 = I * kRowsWG;
  const int ib0 = i0 + 32 * wave;
  const int row = ib0 + l32;
  const float c2 = a.c2;
  const int fbase = frag_base<Op, D>(l32, hh);
  const int tb0 = Op::kConvert ? P::trb_base(lane) : Op::kES == 2 ? trb_base<D>(lane, 0) : 0;
  const int tb1 = !Op::kConvert && Op::kES == 2 ? trb_base<D>(lane, 1) : 0;

  // Key tiles this workgroup sweeps: all of them for the relation; for the cross passes
  // under the causal mask only those holding kept entries (up to the last own row for
  // dA, from the first own row on for dB).  The split divides that range.
  int kt_lo = 0, kt_hi = a.key_tiles;
  if constexpr (CAUSAL && MODE == 1) kt_hi = min(a.key_tiles, (i0 + kRowsWG + kBC - 1) / kBC);
  if constexpr (CAUSAL && MODE == 2) kt_lo = i0 / kBC;
  const int kt_begin = kt_lo + (int)(((int64_t)(kt_hi - kt_lo) * split) / a.splits);
  const int kt_end = kt_lo + (int)(((int64_t)(kt_hi - kt_lo) * (split + 1)) / a.splits);
  const int NB = 2 * (kt_end - kt_begin);

  // bf16 inputs: where the chunks this lane copies go in the fp16 image.  Copy qq of a tile
  // covers rows rq = qq kWave / kCPR .. (a multiple of 4) and the lane takes row rq + l / kCPR,
  // stored chunk l % kCPR, i.e. column chunk (l % kCPR) ^ swz(row).  With 16 chunks per row
  // swz(row) = swz(l / kCPR) ^ (qq % 4) and the image offset of that chunk is this lane's
  // offset for qq = 0, bits 4-5 flipped by qq % 4, plus rq 64; with 8 it is the qq = 0 offset
  // plus rq 64.
  auto img_lane_of = [](int l) __attribute__((always_inline)) {
    return P::off(l / G::kCPR, (l % G::kCPR) ^ G::swz(l / G::kCPR));
  };
  const int img_lane = img_lane_of(lane);
  // Stage: [teacher tile][student tile]([fp16 image])[teacher stats][student stats]; all 8
  // waves copy their share of the two tiles, and waves 0 and 1 the 64 LSE values of the
  // teacher and the student (one per lane, rows beyond N read row N-1).
  auto stage_tile = [&](int k, char* st_base) __attribute__((always_inline)) {
    const int j0 = (kt_begin + k) * kBC;
    if constexpr (CAUSAL) {
      // the tile's base plus per-lane offsets of the clamped row and chunk, held per copy
      // (the non-causal form below, which forms them per copy, measured 1% slower here)
      const int lim = N - 1 - j0;
      const char* tbt = yt_c + (int64_t)j0 * tsn_b;
      const char* tbs = ys_c + (int64_t)j0 * ssn_b;
#pragma unroll
      for (int q = 0; q < kDma; ++q) {
        const int slot0 = (wave * kDma + q) * kWave;
        const int t = slot0 + lane;
        const uint32_t r = (uint32_t)min(t / G::kCPR, lim);
        const uint32_t c16 = (uint32_t)(((t % G::kCPR) ^ G::swz(t / G::kCPR)) * 16);
        lds_copy16_s(__umul24(r, tsn_u24) + c16, tbt, lds_addr(st_base + slot0 * 16));
        lds_copy16_s(__umul24(r, ssn_u24) + c16, tbs, lds_addr(st_base + G::kTileBytes + slot0 * 16));
      }
      if (wave < 2) {
        lds_copy4_s((uint32_t)min(lane, lim) * 4u, (wave == 0 ? stg_t : stg_s) + j0,
                    lds_addr(st_base + kStatsOff + wave * kBC * 4));
      }
    } else {
      const int lim = N - 1 - j0;  // last row of the unit, relative to the tile (>= 0)
      const int xr = lane / G::kCPR;
      const int xc16 = ((lane % G::kCPR) ^ G::swz(xr)) << 4;
#pragma unroll
      for (int q = 0; q < kDma; ++q) {
        const int slot0 = (wave * kDma + q) * kWave;
        // copy q covers rows rb .. rb + 64 / kCPR - 1 of the tile; lane l takes row
        // rb + l / kCPR (clamped to the unit's last row) and chunk l % kCPR, stored at the
        // swizzled slot.  For rb a multiple of 64 / kCPR, swz(rb + x) = swz(rb) ^ swz(x), so
        // the lane's part is the loop-invariant xc16 XOR a uniform constant.
        const int rb = slot0 / G::kCPR;
        const int rq = min(rb, lim);  // uniform; the lane adds min(l / kCPR, lim - rq) rows
        int sq = G::swz(rb) << 4;
        asm volatile("" : "+s"(sq));  // formed per copy: the non-causal sweep has no register
                                      // to hold one offset per copy through the loop
        const uint32_t rr = (uint32_t)min(xr, lim - rq);
        const uint32_t c16 = (uint32_t)(xc16 ^ sq);
        lds_copy16_s(__umul24(rr, tsn_u24) + c16, yt_c + (int64_t)(j0 + rq) * tsn_b,
                     lds_addr(st_base + slot0 * 16));
        lds_copy16_s(__umul24(rr, ssn_u24) + c16, ys_c + (int64_t)(j0 + rq) * ssn_b,
                     lds_addr(st_base + G::kTileBytes + slot0 * 16));
      }
      if (wave < 2) {
        lds_copy4_s((uint32_t)min(lane, lim) * 4u, (wave == 0 ? stg_t : stg_s) + j0,
                    lds_addr(st_base + kStatsOff + wave * kBC * 4));
      }
    }
  };
  // Once a wave's own copies into a stage buffer have completed (wait_vmem): the fp16 image
  // of the student chunks it copied (ImgGeo layout), and, for waves 0 and 1, its
  // LSE values turned into log2 statistics (rows beyond N: a huge value, i.e. R = 0).
  auto convert_tile = [&](int k, char* st_base) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");  // the reads below follow the completed copies
    if constexpr (Op::kConvert) {
      // the non-causal sweep has no register to hold img_lane through: formed here from the
      // lane index, opaque to the compiler
      int il = img_lane;
      if constexpr (!CAUSAL) {
        int ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        il = img_lane_of(ln);
      }
#pragma unroll
      for (int q = 0; q < kDma; ++q) {
        const int qq = wave * kDma + q;  // wave-uniform
        const int off = (qq * kWave + lane) * 16;
        const int io = (il ^ ((G::kCPR >= 16 ? qq & 3 : 0) << 4)) + qq * (kWave / G::kCPR) * 64;
        const u32x4 v = *reinterpret_cast<const u32x4*>(st_base + G::kTileBytes + off);
        *reinterpret_cast<u32x4*>(st_base + kGradOff + io) =
            bf16x8_to_f16x8_bits(__builtin_bit_cast(bf16x8, v));
      }
    }
    if (wave < 2) {
      float* sv = reinterpret_cast<float*>(st_base + kStatsOff) + wave * kBC + lane;
      const int j = (kt_begin + k) * kBC + lane;
      *sv = j < N ? fmaf(*sv, kLog2e, -kWScaleLog2) : kPosBig;
    }
  };
  const int ntiles = NB >> 1;
  // stage buffer of tile t (t >= 0)
  auto buf = [&](int t) __attribute__((always_inline)) { return lds + (t % kStages) * kStage; };
  if (ntiles > 0) stage_tile(0, buf(0));
  // M(0)'s gradient part reads the last buffer's gradient tile before any copy fills it
  for (int q = tid; q < (Op::kConvert ? kImgB : G::kTileBytes) / 16; q += kW * kWave)
    *reinterpret_cast<u32x4*>(buf(kStages - 1) + kGradOff + 16 * q) = u32x4{0u, 0u, 0u, 0u};

  frag_t qt[KS], qs[KS];
  float rt, rs;  // own row statistics
  float wd2 = 0.f;  // 2 (R_s(i,i) - R_t(i,i)) 2^14 of the own row (relation)
  if (row < N) {
    rt = fmaf(own_t[row], kLog2e, -kWScaleLog2);
    rs = fmaf(own_s[row], kLog2e, -kWScaleLog2);
    if (MODE == 0 && a.diag_delta != nullptr)
      wd2 = a.diag_delta[(int64_t)unit * N + row] * (2.0f * 16384.0f);
  } else {
    rt = kPosBig;
    rs = kPosBig;
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (row < N) {
      qt[ks] = load_frag_global<Op>(xt + (int64_t)row * tsn + 16 * ks + 8 * hh);
      qs[ks] = load_frag_global<Op>(xs + (int64_t)row * ssn + 16 * ks + 8 * hh);
    } else {
      qt[ks] = frag_t{};
      qs[ks] = frag_t{};
    }
  }

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
  f32x16 st = f32x16{}, ss = f32x16{};
  gfrag_t wf0 = gfrag_t{}, wf1 = gfrag_t{};

  auto block_j0 = [&](int n) { return (kt_begin + (n >> 1)) * kBC + 32 * (n & 1); };

  // Every wave runs M(n) then V(n) for its own rows; the two waves of a SIMD drift freely,
  // so one wave's exp/VALU work overlaps the other's MFMAs and both keep LDS reads in
  // flight.  Barriers only separate key tiles (two blocks each):
  //  * three buffers: step t copies tile t+1 into the buffer of tile t-2 (last read in
  //    step t-1) at its start and awaits it at its end;
  //  * two buffers (fp32, d = 128): tile t+1 goes into the buffer of tile t-1, whose last
  //    reads are the gradient MFMAs of M(2t); a barrier after M(2t) precedes the copy.
  // The barrier ending step t publishes tile t+1 (its fp16 image and statistics made by
  // each wave after M(2t) from the chunks it copied) to every wave.  A V(2t-1) that a wave
  // runs at the start of step t (below) reads tile t-1's statistics before either copy
  // reaches them.

  // M(n): gradient of block n-1, scores of block n.  Every M runs the full pipeline: M(0)
  // contracts the initial zero W with the zero-filled gradient tile of the last buffer;
  // blocks at or beyond N contract a zero W (V leaves zero fragments) with finite copies
  // of row N-1 and their scores are never used; M(NB) computes unused scores from a buffer
  // no copy is writing into.
  auto m_phase = [&](int n) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);  // matrix phases issue ahead of a partner's vector work
    const char* sb = buf(n >> 1);
    const char* gtile = (n == 0 ? buf(kStages - 1) : buf((n - 1) >> 1)) + kGradOff;
    const int jbg = 32 * ((n - 1) & 1), jbs = n & 1;
    m_pipeline<Op, D>(gtile, jbg, sb, jbs, fbase, lane, tb0, tb1, wf0, wf1, qt, qs, acc, st, ss);
  };

  // V(n): W(n) from the scores of block n and the column statistics staged with its tile.
  // hhp, rowp: the lane's half-wave index and row as the non-causal kernel's last call forms
  // them again (below); the causal kernel uses the values it holds
  auto v_phase = [&](int n, int hhp, int rowp) __attribute__((always_inline)) {
    const int hh_ = CAUSAL ? hh : hhp, row_ = CAUSAL ? row : rowp;
    __builtin_amdgcn_s_setprio(0);
    const char* sb = buf(n >> 1);
    const int jb0 = block_j0(n);
    if (jb0 < N) {
      const int jb = n & 1;
      const float* clt = reinterpret_cast<const float*>(sb + kStatsOff) + 32 * jb;
      const float* cls = clt + kBC;
      f32x8 w32[2];
      const int di = row_ - jb0;
      const int nl = N - jb0;
      const bool tail = jb0 + 32 > N;
      constexpr bool ROW = MODE != 2, COL = MODE != 1, SUB = MODE == 0;
      bool none = false;  // the block holds no entry this pass keeps
      if constexpr (!CAUSAL) {
        if (SUB && jb0 == ib0) {  // the wave's diagonal block
          if (tail) make_w<ROW, COL, false, true, SUB>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
          else make_w<ROW, COL, false, false, SUB>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
        } else if (tail) {
          make_w<ROW, COL, false, true>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
        } else {
          make_w<ROW, COL, false, false>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
        }
      } else {
        if (jb0 + 31 < ib0) {  // strictly below the diagonal: row terms
          if constexpr (ROW) make_w<true, false, false, false>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
          else none = true;
        } else if (jb0 > ib0 + 31) {  // strictly above: column terms
          if constexpr (COL) {
            if (tail) make_w<false, true, false, true>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
            else make_w<false, true, false, false>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
          } else {
            none = true;
          }
        } else {
          if (tail) make_w<ROW, COL, true, true, SUB>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
          else make_w<ROW, COL, true, false, SUB>(st, ss, rt, rs, clt, cls, hh_, di, nl, c2, wd2, w32);
        }
      }
      if (none) {
        wf0 = gfrag_t{};
        wf1 = gfrag_t{};
      } else {
        wf0 = w_frag<Op>(w32[0]);
        wf1 = w_frag<Op>(w32[1]);
      }
    } else {
      wf0 = gfrag_t{};
      wf1 = gfrag_t{};
    }
  };

  // Waves w and w + 4 share a SIMD.  The barrier that ends each step would start both in their
  // matrix phases; waves 4-7 instead run V of a tile's last block after the barrier, at the
  // start of the next step, so their matrix phases fall beside the vector phases of waves 0-3
  // (each wave's own order of operations is unchanged; its stage buffer is still resident).
  const bool lag = kW == 8 && wave >= 4;
  wait_vmem();
  if (ntiles > 0) convert_tile(0, buf(0));
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (kStages == 3 && t + 1 < ntiles) stage_tile(t + 1, buf(t + 1));
    if (lag && t > 0) v_phase(2 * t - 1, hh, row);
    m_phase(2 * t);
    if (kStages == 2) {
      lds_barrier();
      if (t + 1 < ntiles) stage_tile(t + 1, buf(t + 1));
    }
    if (kStages == 3) {
      // tile t+1's copies, issued at the start of this step, have usually landed by now:
      // its fp16 image and statistics are made here, beside the partner wave's work, rather
      // than just before the barrier
      wait_vmem();
      if (t + 1 < ntiles) convert_tile(t + 1, buf(t + 1));
    }
    v_phase(2 * t, hh, row);
    m_phase(2 * t + 1);
    if (!lag) v_phase(2 * t + 1, hh, row);
    wait_vmem();
    if (kStages == 2 && t + 1 < ntiles) convert_tile(t + 1, buf(t + 1));
    lds_barrier();
  }
  if (lag && ntiles > 0) {
    // the non-causal sweep leaves no register for the lane's indices to survive the loop
    // in: this last call forms them again (opaque to the compiler)
    if constexpr (CAUSAL) {
      v_phase(NB - 1, hh, row);
    } else {
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      v_phase(NB - 1, ln >> 5, ib0 + (ln & 31));
    }
  }
  m_phase(NB);

  // Scale and write: acc[mb][r] = dX[i][d] * 2^14 / (scale g) for
  // i = ib0 + 8 (r/4) + 4 hh + (r%4), d = 32 mb + l32.
  const float factor = a.scale * a.grad_loss[0] * (1.0f / 16384.0f);
  // the lane's indices again, formed here (opaque to the compiler) so that none of the
  // epilogue's lane-derived values has to be held through the sweep
  int lne = lane;
  if constexpr (!CAUSAL)
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lne));
  const int l32e = CAUSAL ? l32 : lne & 31, hhe = CAUSAL ? hh : lne >> 5;
  if (a.rope_cos != nullptr) {
    // Gradient before the student's rotation: the transposed rotate-half rotation maps
    // (g_k, g_{k+D/2}) to (g_k c + g_{k+D/2} s, g_{k+D/2} c - g_k s) with the cos / sin of
    // row i, frequency k.  Dimensions k and k + D/2 sit in blocks mb and mb + MB/2 of
    // the same lane.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = ib0 + 8 * (r >> 2) + 4 * hhe + (r & 3);
      if (i >= N) continue;
#pragma unroll
      for (int mb = 0; mb < MB / 2; ++mb) {
        const int64_t t = (int64_t)i * (D / 2) + 32 * mb + l32e;
        const float c = a.rope_cos[t], sn = a.rope_sin[t];
        const float g1 = acc[mb][r], g2 = acc[mb + MB / 2][r];
        acc[mb][r] = fmaf(g1, c, g2 * sn);
        acc[mb + MB / 2][r] = fmaf(g2, c, -(g1 * sn));
      }
    }
  }
  if (a.splits == 1) {
    const bool full = ib0 + 32 <= N;
    char* gbase = reinterpret_cast<char*>(a.dx) + (b * a.g_sb + hin * a.g_sh) * (OUT_F32 ? 4 : 2);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = ib0 + 8 * (r >> 2) + 4 * hhe + (r & 3);
      if (!full && i >= N) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int64_t o = (int64_t)i * a.g_sn + 32 * mb + l32e;
        const float v = acc[mb][r] * factor;
        if constexpr (OUT_F32)
          reinterpret_cast<float*>(gbase)[o] = v;
        else
          reinterpret_cast<uint16_t*>(gbase)[o] = f32_to_bf16_rne(v);
      }
    }
  } else {
    const int rows_pad = a.row_tiles * kRowsWG;
    float* dst = a.partial + ((int64_t)split * a.B * a.H + unit) * rows_pad * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = ib0 + 8 * (r >> 2) + 4 * hhe + (r & 3);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) dst[(int64_t)i * D + 32 * mb + l32e] = acc[mb][r] * factor;
    }
  }
}

// Fixed-order sum of the split-K partials into the gradient (one thread per 4 d-values).
template <bool OUT_F32>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const ReduceLaunch L) {
  const int mi = member_of(L, (int)blockIdx.x);
  const ReduceArgs& a = L.m[mi];
  const int64_t q = (int64_t)((int)blockIdx.x - member_begin(L, mi)) * 256 + threadIdx.x;
  const int dq = a.d / 4;
  const int64_t total = (int64_t)a.B * a.H * a.N * dq;
  if (q >= total) return;
  const int c4 = (int)(q % dq);
  const int64_t rowlin = q / dq;
  const int i = (int)(rowlin % a.N);
  const int unit = (int)(rowlin / a.N);
  const int b = unit / a.H, h = unit % a.H;
  const int hin = head_of(L, a.map_off, h);
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < a.splits; ++c) {
    const float* p = a.partial + (((int64_t)c * a.B * a.H + unit) * a.rows_pad + i) * a.d + 4 * c4;
    s += *reinterpret_cast<const f32x4*>(p);
  }
  const int64_t o = b * a.g_sb + hin * a.g_sh + (int64_t)i * a.g_sn + 4 * c4;
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.dx) + o) = s;
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.dx) + o;
    const uint32_t lo = (uint32_t)f32_to_bf16_rne(s[0]) | ((uint32_t)f32_to_bf16_rne(s[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_rne(s[2]) | ((uint32_t)f32_to_bf16_rne(s[3]) << 16);
    *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
  }
}

// ------------------------------------------------------------------ RoPE prep
// Rotated copies of the teacher and student rows for the RoPE-fused and cross entry points:
// for token p and frequency k < D/2 (rotate-half pairing of k with k + D/2)
//   y_k = x_k cos[p][k] - x_{k+D/2} sin[p][k],   y_{k+D/2} = x_{k+D/2} cos[p][k] + x_k sin[p][k]
// rounded once to the input dtype (nearest even), as the rotation inside the model would
// leave it.  Each product of a bf16 or fp32 element with an fp32 table entry is exact in
// fp64, so the fp64 sum below is the exact rotation rounded once to fp64, and the dtype's
// rounding is taken from it directly.  F16_IMAGES stores each bf16 value as the exactly
// equal IEEE fp16 value (the cross relation's matrix-core operands).  Written into the
// reserve, dense [unit][N][D]; a side without tables is copied unrotated.  One thread per
// (side, unit, row, group of 4 frequencies): consecutive threads cover consecutive
// frequencies of one row, so each half-row is read and written in one run.

// Nearest-even bf16 bits of an fp64 value (finite, within the bf16 range): the significand
// is rounded at bit 45 (7 stored bits remain) on the fp64 bit pattern, after which the
// value is exact in fp32 and its top half is the bf16 pattern.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t low = (1ull << 45) - 1;       // the 45 bits rounded off
  u += ((1ull << 44) - 1) + ((u >> 45) & 1ull);  // half a unit, ties to the even side
  u &= ~low;
  return (uint16_t)(__float_as_uint((float)__longlong_as_double((long long)u)) >> 16);
}

template <bool IN_BF16, int D, bool F16_IMAGES>
__global__ __launch_bounds__(256) void rope_prep_kernel(const PrepLaunch L) {
  constexpr int G4 = D / 8;  // groups of 4 frequencies per row
  const int mi = member_of(L, (int)blockIdx.x);
  const PrepArgs& a = L.m[mi];
  const int64_t q = (int64_t)((int)blockIdx.x - member_begin(L, mi)) * 256 + threadIdx.x;
  const int64_t per_side = (int64_t)a.B * a.H * a.N * G4;
  if (q >= 2 * per_side) return;
  const int side = (int)(q / per_side);
  const int64_t rq = q - side * per_side;
  const int g = (int)(rq % G4);
  const int64_t rowlin = rq / G4;
  const int p = (int)(rowlin % a.N);
  const int unit = (int)(rowlin / a.N);
  const int b = unit / a.H, h = unit % a.H;
  const int hin = head_of(L, a.map_off, h);
  const void* x = side ? a.x_s : a.x_t;
  const int64_t sb = side ? a.s_sb : a.t_sb, sh = side ? a.s_sh : a.t_sh;
  const int64_t sn = side ? a.s_sn : a.t_sn;
  const float* cs = side ? a.cos_s : a.cos_t;
  const float* sn_tab = side ? a.sin_s : a.sin_t;
  const int64_t src = b * sb + hin * sh + (int64_t)p * sn + 4 * g;
  f32x4 x1, x2;
  if constexpr (IN_BF16) {
    const uint16_t* xp = reinterpret_cast<const uint16_t*>(x) + src;
    const u32x2 v1 = *reinterpret_cast<const u32x2*>(xp);
    const u32x2 v2 = *reinterpret_cast<const u32x2*>(xp + D / 2);
    x1 = f32x4{__uint_as_float(v1[0] << 16), __uint_as_float(v1[0] & 0xffff0000u),
               __uint_as_float(v1[1] << 16), __uint_as_float(v1[1] & 0xffff0000u)};
    x2 = f32x4{__uint_as_float(v2[0] << 16), __uint_as_float(v2[0] & 0xffff0000u),
               __uint_as_float(v2[1] << 16), __uint_as_float(v2[1] & 0xffff0000u)};
  } else {
    const float* xp = reinterpret_cast<const float*>(x) + src;
    x1 = *reinterpret_cast<const f32x4*>(xp);
    x2 = *reinterpret_cast<const f32x4*>(xp + D / 2);
  }
  double y1[4], y2[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y1[e] = (double)x1[e];
    y2[e] = (double)x2[e];
  }
  if (cs != nullptr) {
    const int64_t t = (int64_t)p * (D / 2) + 4 * g;
    const f32x4 c = *reinterpret_cast<const f32x4*>(cs + t);
    const f32x4 sv = *reinterpret_cast<const f32x4*>(sn_tab + t);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // exact products, one rounding of their difference / sum
      const double p11 = (double)x1[e] * (double)c[e], p22 = (double)x2[e] * (double)sv[e];
      const double p21 = (double)x2[e] * (double)c[e], p12 = (double)x1[e] * (double)sv[e];
      y1[e] = p11 - p22;
      y2[e] = p21 + p12;
    }
  }
  const int64_t dst = ((int64_t)unit * a.N + p) * D + 4 * g;
  if constexpr (IN_BF16) {
    uint16_t* cp = reinterpret_cast<uint16_t*>(side ? a.c_s : a.c_t) + dst;
    uint16_t h1[4], h2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h1[e] = f64_to_bf16_rne(y1[e]);
      h2[e] = f64_to_bf16_rne(y2[e]);
    }
    if constexpr (F16_IMAGES) {  // the bf16 values as fp16 bit patterns (exact below 65504)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v1 = __uint_as_float((uint32_t)h1[e] << 16);
        const float v2 = __uint_as_float((uint32_t)h2[e] << 16);
        h1[e] = __builtin_bit_cast(uint16_t, (_Float16)v1);
        h2[e] = __builtin_bit_cast(uint16_t, (_Float16)v2);
      }
    }
    *reinterpret_cast<u32x2*>(cp) =
        u32x2{(uint32_t)h1[0] | ((uint32_t)h1[1] << 16), (uint32_t)h1[2] | ((uint32_t)h1[3] << 16)};
    *reinterpret_cast<u32x2*>(cp + D / 2) =
        u32x2{(uint32_t)h2[0] | ((uint32_t)h2[1] << 16), (uint32_t)h2[2] | ((uint32_t)h2[3] << 16)};
  } else {
    float* cp = reinterpret_cast<float*>(side ? a.c_s : a.c_t) + dst;
    *reinterpret_cast<f32x4*>(cp) = f32x4{(float)y1[0], (float)y1[1], (float)y1[2], (float)y1[3]};
    *reinterpret_cast<f32x4*>(cp + D / 2) =
        f32x4{(float)y2[0], (float)y2[1], (float)y2[2], (float)y2[3]};
  }
}

// ------------------------------------------------------------------ launchers
static bool fault_injected() {
  const char* v = getenv("LARD_FAULT_INJECT");
  return v && v[0] == '1';
}

template <class M>
static int grid_of(const Launch<M>& L) {
  return L.n >= 1 ? L.end[L.n - 1] : 0;
}

template <class In, int D, bool CAUSAL, bool REL>
static int launch_fwd_t(const FwdLaunch& a, const LossOut& loss, hipStream_t s) {
  hipLaunchKernelGGL((relkl_fwd_kernel<In, D, CAUSAL, REL>), dim3(grid_of(a)), dim3(kThreads),
                     0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1 + loss.n), dim3(256), 0, s, loss);
  return (int)hipGetLastError();
}

template <class In, bool REL>
static int launch_fwd_d(const FwdLaunch& a, int d, bool causal, const LossOut& loss,
                        hipStream_t s) {
  if (d == 128) return causal ? launch_fwd_t<In, 128, true, REL>(a, loss, s)
                              : launch_fwd_t<In, 128, false, REL>(a, loss, s);
  return causal ? launch_fwd_t<In, 64, true, REL>(a, loss, s)
                : launch_fwd_t<In, 64, false, REL>(a, loss, s);
}

int launch_fwd(const FwdLaunch& a, bool in_bf16, int d, bool causal, const LossOut& loss,
               void* stream, bool cross) {
  if (fault_injected()) return (int)hipErrorLaunchFailure;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (cross) {
    return in_bf16 ? launch_fwd_d<F16Op, false>(a, d, causal, loss, s)
                   : launch_fwd_d<F32In, false>(a, d, causal, loss, s);
  }
  return in_bf16 ? launch_fwd_d<Bf16In, true>(a, d, causal, loss, s)
                 : launch_fwd_d<F32In, true>(a, d, causal, loss, s);
}

template <class Op, int D, bool CAUSAL, bool OUT_F32, int MODE>
static int launch_bwd_t(const BwdLaunch& a, hipStream_t s) {
  hipLaunchKernelGGL((relkl_bwd_kernel<Op, D, CAUSAL, OUT_F32, MODE>), dim3(grid_of(a)),
                     dim3(bwd_waves(Op::kES == 4) * kWave), 0, s, a);
  return (int)hipGetLastError();
}

template <class Op, int D, int MODE>
static int launch_bwd_d(const BwdLaunch& a, bool causal, bool out_f32, hipStream_t s) {
  if (causal) return out_f32 ? launch_bwd_t<Op, D, true, true, MODE>(a, s)
                             : launch_bwd_t<Op, D, true, false, MODE>(a, s);
  return out_f32 ? launch_bwd_t<Op, D, false, true, MODE>(a, s)
                 : launch_bwd_t<Op, D, false, false, MODE>(a, s);
}

template <int MODE>
static int launch_bwd_m(const BwdLaunch& a, bool in_bf16, int d, bool causal, bool out_f32,
                        hipStream_t s) {
  // the relation reads bf16 rows (in place or rotated copies); the cross relation the
  // reserve's fp16 images
  using Op16 = std::conditional_t<MODE == 0, Bf16Op, F16Op>;
  if (in_bf16) {
    return d == 128 ? launch_bwd_d<Op16, 128, MODE>(a, causal, out_f32, s)
                    : launch_bwd_d<Op16, 64, MODE>(a, causal, out_f32, s);
  }
  // fp32 inputs always give an fp32 gradient
  return d == 128 ? launch_bwd_d<F32In, 128, MODE>(a, causal, true, s)
                  : launch_bwd_d<F32In, 64, MODE>(a, causal, true, s);
}

int launch_bwd(const BwdLaunch& a, bool in_bf16, int d, bool causal, bool out_f32, void* stream,
               int mode) {
  if (fault_injected()) return (int)hipErrorLaunchFailure;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (mode == 1) return launch_bwd_m<1>(a, in_bf16, d, causal, out_f32, s);
  if (mode == 2) return launch_bwd_m<2>(a, in_bf16, d, causal, out_f32, s);
  return launch_bwd_m<0>(a, in_bf16, d, causal, out_f32, s);
}

int launch_rope_prep(const PrepLaunch& a, bool in_bf16, int d, void* stream, bool f16_images) {
  if (fault_injected()) return (int)hipErrorLaunchFailure;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(grid_of(a));
  if (in_bf16 && f16_images) {
    if (d == 128) hipLaunchKernelGGL((rope_prep_kernel<true, 128, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rope_prep_kernel<true, 64, true>), grid, dim3(256), 0, s, a);
  } else if (in_bf16) {
    if (d == 128) hipLaunchKernelGGL((rope_prep_kernel<true, 128, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rope_prep_kernel<true, 64, false>), grid, dim3(256), 0, s, a);
  } else {
    if (d == 128) hipLaunchKernelGGL((rope_prep_kernel<false, 128, false>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((rope_prep_kernel<false, 64, false>), grid, dim3(256), 0, s, a);
  }
  return (int)hipGetLastError();
}


int launch_splitk_reduce(const ReduceLaunch& a, bool out_f32, void* stream) {
  if (fault_injected()) return (int)hipErrorLaunchFailure;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (out_f32)
    hipLaunchKernelGGL(splitk_reduce_kernel<true>, dim3(grid_of(a)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<false>, dim3(grid_of(a)), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

}  // namespace lard
