// Internal interface between the C-ABI layer (lard_api.cpp) and the HIP kernels
// (relkl_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lard.h"

namespace lard {

// Work decomposition shared by host sizing and device kernels.
constexpr int kWave = 64;
constexpr int kWaves = 4;                 // waves per workgroup (two workgroups per CU)
constexpr int kThreads = kWave * kWaves;  // 256
constexpr int kBR = kWaves * 32;          // forward rows per workgroup: 32 per wave
constexpr int kBC = 64;                   // rows of one key tile staged in LDS
// Backward workgroup: 8 waves (two per SIMD, 256 rows) for 2-byte operands; 4 waves (one
// per SIMD, 128 rows) for fp32, whose operands take twice the registers: one wave per SIMD
// may use 512 (vector and accumulator registers together) instead of 256.
constexpr int bwd_waves(bool f32) { return f32 ? 4 : 8; }
constexpr int bwd_rows(bool f32) { return 32 * bwd_waves(f32); }

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Caller-owned "reserve" of the RoPE-fused and cross entry points: the rotated (or copied)
// rows the kernels read in place of the caller's tensors, dense [units][N][d] per matrix:
// x_t, x_s (the relation's rows, or the cross relation's A) and, for the cross relation,
// y_t, y_s (its B).  Elements are copy_bytes wide: the input dtype for the relation (bf16 or
// fp32), fp16 images of the bf16 values (or fp32) for the cross relation.  The plain entry
// points need no reserve: the forward's per-row outputs are the whole state.
struct ReserveLayout {
  size_t x_t, x_s, y_t, y_s, total;
};

inline ReserveLayout reserve_layout(int64_t units, int64_t N, int64_t d, int copy_bytes,
                                    bool cross = false) {
  ReserveLayout L;
  const size_t copy = (size_t)round_up(units * N * d * copy_bytes, 256);
  L.x_t = 0;
  L.x_s = copy;
  L.y_t = cross ? 2 * copy : L.x_t;
  L.y_s = cross ? 3 * copy : L.x_s;
  L.total = (cross ? 4 : 2) * copy;
  return L;
}

struct FwdArgs {
  const void* x_t;    // own (query-side) rows
  const void* x_s;
  const void* y_t;    // key-side rows with x's layout (cross relation), or null: x itself
  const void* y_s;
  int64_t t_sb, t_sh, t_sn;
  int64_t s_sb, s_sh, s_sn;
  int32_t B, H, N;
  int32_t row_tiles;  // ceil(N / kBR)
  float scale;        // logit scale
  float c2;           // scale * log2(e)
  float* lse_t;
  float* lse_s;
  float* row_kl;      // may be null
  float* diag_delta;  // R_s(i,i) - R_t(i,i) per row (the relation; null for the cross relation)
  double* partial;    // [B*H*row_tiles]
  int32_t map_off;    // head map: offset in the launch's table, or -1 (identity)
};

struct BwdArgs {
  const void* x_t;    // own rows: the caller's tensors (strides below) or dense copies
  const void* x_s;
  const void* y_t;    // staged rows with x_dense (cross relation: the other matrix; the
  const void* y_s;    // relation: x)
  int64_t t_sb, t_sh, t_sn;
  int64_t s_sb, s_sh, s_sn;
  int64_t g_sb, g_sh, g_sn;  // gradient strides (elements)
  int32_t B, H, N;
  int32_t row_tiles;   // ceil(N / bwd_rows)
  int32_t key_tiles;   // ceil(N / kBC)
  int32_t splits;      // split-K count over key tiles
  float scale;
  float c2;
  const float* lse_t;     // the forward's LSE (nats, dense [units][N]) of the own rows
  const float* lse_s;
  const float* lc_t;      // ... and of the staged rows (the same for the relation; the
  const float* lc_s;      // cross relation's query rows in both of its passes)
  const float* diag_delta;  // R_s(i,i) - R_t(i,i) per own row (relation), or null
  const float* grad_loss;
  const float* rope_cos;  // student RoPE tables [N][d/2] (fused entry points) or null:
  const float* rope_sin;  // the gradient is rotated back before it is written
  int32_t x_dense;        // x_* / y_* are dense [unit][N][d] copies (else x_* in place)
  void* dx;            // final gradient (splits == 1)
  float* partial;      // [splits][B*H][row_tiles*bwd_rows][d] (splits > 1)
  int32_t map_off;
};

// Rotation of the inputs into the reserve for the RoPE-fused entry points.
struct PrepArgs {
  const void* x_t;
  const void* x_s;
  int64_t t_sb, t_sh, t_sn;
  int64_t s_sb, s_sh, s_sn;
  int32_t B, H, N;
  const float* cos_t;  // [N][d/2] tables, or null (side not rotated)
  const float* sin_t;
  const float* cos_s;
  const float* sin_s;
  void* c_t;           // reserve copies, dense [units][N][d]
  void* c_s;
  int32_t map_off;
};

struct ReduceArgs {
  const float* partial;
  void* dx;
  int64_t g_sb, g_sh, g_sn;
  int32_t B, H, N, d;
  int32_t rows_pad;    // row_tiles * bwd_rows
  int32_t splits;
  int32_t map_off;
};

// One launch covers up to kMaxGroup members (relation problems that share the dtype, d and
// mask, e.g. Q/Q on the query heads and K/K, V/V on the KV heads of one layer).  The grid
// is the members' workgroups (or blocks) back to back: member k takes [end[k-1], end[k]).
// Head maps of all members sit in one table; member k's entries start at m[k].map_off.
constexpr int kMaxGroup = LARD_MAX_GROUP;
constexpr int kMapSlots = 512;

template <class M>
struct Launch {
  M m[kMaxGroup];
  int32_t n;
  int32_t end[kMaxGroup];
  int16_t head_map[kMapSlots];
};
using FwdLaunch = Launch<FwdArgs>;
using BwdLaunch = Launch<BwdArgs>;
using PrepLaunch = Launch<PrepArgs>;
using ReduceLaunch = Launch<ReduceArgs>;
static_assert(sizeof(BwdLaunch) <= 4096 && sizeof(FwdLaunch) <= 4096,
              "a launch's arguments must fit the 4 KiB kernel-argument segment");

// Where the forward's per-workgroup loss partials go: `total` receives the sum over every
// member, member[k] (when non-null) the sum over member k's workgroups [begin[k],
// begin[k+1]).  The partials of all members are contiguous.
struct LossOut {
  const double* partial;
  float* total;
  float* member[kMaxGroup];
  int32_t begin[kMaxGroup + 1];
  int32_t n;
};

// Each returns a hipError_t value (0 on success).  `in_bf16`: input dtype; `out_f32`:
// gradient dtype (fp32 or the input dtype).
// cross: the cross relation (own rows and key rows from different matrices; no diagonal
// reference; bf16 inputs arrive as the reserve's fp16 images).
int launch_fwd(const FwdLaunch& a, bool in_bf16, int d, bool causal, const LossOut& loss,
               void* stream, bool cross = false);
// mode: 0 relation gradient, 1 cross dA pass, 2 cross dB pass (see relkl_bwd_kernel).
int launch_bwd(const BwdLaunch& a, bool in_bf16, int d, bool causal, bool out_f32,
               void* stream, int mode = 0);
int launch_splitk_reduce(const ReduceLaunch& a, bool out_f32, void* stream);
// f16_images: write bf16 rows as their fp16 images (cross relation), else in the input dtype.
int launch_rope_prep(const PrepLaunch& a, bool in_bf16, int d, void* stream, bool f16_images);

// Capacity (fp64 loss partials, one per forward workgroup) of the library-owned scratch of
// the allocation-free forward, and its device address on the current device (a hipError_t
// value, 0 on success; looked up once per device).
constexpr int64_t kNoallocMaxPartials = LARD_NOALLOC_MAX_PARTIALS;
int scratch_address(void** out);

}  // namespace lard
