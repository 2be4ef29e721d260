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
constexpr int kBWaves = 8;                // backward waves per workgroup (two groups of 4)
constexpr int kBRB = kBWaves * 32;        // backward rows per workgroup
constexpr int kBC = 64;                   // rows of one key tile staged in LDS

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Phase-1 state the forward leaves for the backward ("reserve"), per relation head unit:
//  * copies of the teacher and student rows, dense [units][N][d] each: IEEE fp16 copies
//    of bf16 inputs (the backward's operands; bf16 -> fp16 is exact for
//    2^-17 <= |x| < 65504), and for the RoPE-fused entry points the rotated rows, in fp16
//    (bf16 inputs) or fp32 (fp32 inputs); none for fp32 inputs otherwise;
//  * row statistics in log2 units, r = log2(sum_j 2^(S_ij c2 + b_i)) - b_i - 14, dense
//    [units][Npad] with Npad = N rounded up to kBC, for teacher and student, so that
//    R(i, j) * 2^14 = exp2(S_ij c2 - r_i).
struct ReserveLayout {
  size_t x16_t, x16_s, y16_t, y16_s, r_t, r_s, total;
  int64_t npad;
};

// copy_bytes: bytes per element of the row copies (0: none, 2: fp16, 4: fp32); cross: the
// key-side matrices get copies too (y16_*), otherwise y16_* equal x16_*.
inline ReserveLayout reserve_layout(int64_t units, int64_t N, int64_t d, int copy_bytes,
                                    bool cross = false) {
  ReserveLayout L;
  L.npad = round_up(N, kBC);
  const size_t copy = (size_t)round_up(units * N * d * copy_bytes, 256);
  const size_t stats = (size_t)round_up(units * L.npad * 4, 256);
  const size_t ncopy = cross ? 4 : 2;
  L.x16_t = 0;
  L.x16_s = copy;
  L.y16_t = cross ? 2 * copy : L.x16_t;
  L.y16_s = cross ? 3 * copy : L.x16_s;
  L.r_t = ncopy * copy;
  L.r_s = ncopy * copy + stats;
  L.total = ncopy * copy + 2 * stats;
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
  int32_t npad;       // reserve statistics stride per unit
  float scale;        // logit scale
  float c2;           // scale * log2(e)
  float* lse_t;
  float* lse_s;
  float* row_kl;      // may be null
  double* partial;    // [B*H*row_tiles]
  uint16_t* x16_t;    // reserve fp16 copies (bf16 inputs) or null
  uint16_t* x16_s;
  float* r_t;         // reserve log2 statistics
  float* r_s;
  int32_t map_off;    // head map: offset in the launch's table, or -1 (identity)
};

struct BwdArgs {
  const void* x_t;    // own rows (read by the fp32 path)
  const void* x_s;
  const void* y_t;    // staged rows, fp32 path with x_unit_dense (cross relation: the other
  const void* y_s;    // matrix; the relation: x)
  int64_t t_sb, t_sh, t_sn;
  int64_t s_sb, s_sh, s_sn;
  int64_t g_sb, g_sh, g_sn;  // gradient strides (elements)
  int32_t B, H, N;
  int32_t row_tiles;   // ceil(N / kBRB)
  int32_t key_tiles;   // ceil(N / kBC)
  int32_t splits;      // split-K count over key tiles
  int32_t npad;
  float scale;
  float c2;
  const uint16_t* x16_t;  // reserve fp16 copies of the own rows (bf16 path)
  const uint16_t* x16_s;
  const uint16_t* y16_t;  // ... and of the staged rows (the same for the relation)
  const uint16_t* y16_s;
  const float* r_t;       // log2 statistics of the own rows
  const float* r_s;
  const float* rc_t;      // ... and of the staged rows (the same for the relation)
  const float* rc_s;
  const float* grad_loss;
  const float* rope_cos;  // student RoPE tables [N][d/2] (fused entry points) or null:
  const float* rope_sin;  // the gradient is rotated back before it is written
  int32_t x_unit_dense;   // fp32 path: x_t / x_s are dense [unit][N][d] copies
  void* dx;            // final gradient (splits == 1)
  float* partial;      // [splits][B*H][row_tiles*kBRB][d] (splits > 1)
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
  int32_t rows_pad;    // row_tiles * kBRB
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
// f16_copies: the inputs are the reserve's fp16 copies (RoPE-fused path, bf16 inputs).
int launch_fwd(const FwdLaunch& a, bool in_bf16, int d, bool causal, const LossOut& loss,
               void* stream, bool f16_copies = false);
// mode: 0 relation gradient, 1 cross dA pass, 2 cross dB pass (see relkl_bwd_kernel).
int launch_bwd(const BwdLaunch& a, bool in_bf16, int d, bool causal, bool out_f32,
               void* stream, int mode = 0);
int launch_splitk_reduce(const ReduceLaunch& a, bool out_f32, void* stream);
int launch_rope_prep(const PrepLaunch& a, bool in_bf16, int d, void* stream);

}  // namespace lard
