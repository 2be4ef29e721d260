// Internal interface between the C-ABI layer (lard_api.cpp) and the HIP kernels
// (relkl_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "lard.h"

namespace lard {

// Work decomposition shared by host sizing and device kernels.
constexpr int kWave = 64;
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = kWave * kWaves;  // 256
constexpr int kRowBlocks = 2;             // 32-row blocks held by one wave
constexpr int kRowsPerWave = 32 * kRowBlocks;
constexpr int kBR = kWaves * kRowsPerWave;  // rows of one row tile (256)
constexpr int kBC = 64;                     // rows of one key tile staged in LDS

struct UnitMap {
  int32_t head_map[LARD_MAX_HEADS];
};

struct FwdArgs {
  const void* x_t;
  const void* x_s;
  int64_t t_sb, t_sh, t_sn;
  int64_t s_sb, s_sh, s_sn;
  int32_t B, H, N;
  int32_t row_tiles;  // ceil(N / kBR)
  float scale;        // logit scale
  float c2;           // scale * log2(e)
  float* lse_t;
  float* lse_s;
  float* row_kl;      // may be null
  double* partial;    // [B*H*row_tiles]
  UnitMap map;
};

struct BwdArgs {
  const void* x_t;
  const void* x_s;
  int64_t t_sb, t_sh, t_sn;
  int64_t s_sb, s_sh, s_sn;
  int64_t g_sb, g_sh, g_sn;  // gradient strides (elements)
  int32_t B, H, N;
  int32_t row_tiles;
  int32_t key_tiles;   // ceil(N / kBC)
  int32_t splits;      // split-K count over key tiles
  float scale;
  float c2;
  const float* lse_t;
  const float* lse_s;
  const float* grad_loss;
  void* dx;            // final gradient (splits == 1)
  float* partial;      // [splits][B*H][row_tiles*kBR][d] (splits > 1)
  UnitMap map;
};

struct ReduceArgs {
  const float* partial;
  void* dx;
  int64_t g_sb, g_sh, g_sn;
  int32_t B, H, N, d;
  int32_t rows_pad;    // row_tiles * kBR
  int32_t splits;
  UnitMap map;
};

// Each returns a hipError_t value (0 on success).  `in_bf16`: input dtype; `out_f32`:
// gradient dtype (fp32 or the input dtype).
int launch_fwd(const FwdArgs& a, bool in_bf16, int d, bool causal, float* loss,
               void* stream);
int launch_bwd(const BwdArgs& a, bool in_bf16, int d, bool causal, bool out_f32,
               void* stream);
int launch_splitk_reduce(const ReduceArgs& a, bool out_f32, bool out_bf16_ok, void* stream);

}  // namespace lard
