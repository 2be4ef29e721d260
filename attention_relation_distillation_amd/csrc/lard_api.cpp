// C ABI of the relation-KL library: host-side validation, workspace sizing and launch
// configuration.  Every check runs before the first HIP call, so an invalid request never
// touches the device.  The operation itself is documented in include/lard.h.

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "lard.h"
#include "relkl_internal.h"

namespace {

using namespace lard;

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr int kTargetWorkgroups = 512;  // two rounds of one backward workgroup per CU
constexpr int kMaxSplits = 64;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_size(int dtype) { return dtype == LARD_BF16 ? 2 : 4; }

lard_status check_strides(int dtype, int64_t sb, int64_t sh, int64_t sn) {
  const int64_t q = 16 / elem_size(dtype);
  if (sb < 0 || sh < 0 || sn < 0) return LARD_ERR_INVALID_ARGUMENT;
  if (sb % q || sh % q || sn % q) return LARD_ERR_INVALID_ARGUMENT;
  return LARD_OK;
}

lard_status check_desc(const lard_relkl_desc* d) {
  if (!d) return LARD_ERR_INVALID_ARGUMENT;
  if (d->dtype != LARD_FP32 && d->dtype != LARD_BF16) return LARD_ERR_INVALID_ARGUMENT;
  if (d->B < 1 || d->H_in < 1 || d->N < 1 || d->d < 1) return LARD_ERR_INVALID_ARGUMENT;
  if (d->d != 64 && d->d != 128) return LARD_ERR_UNSUPPORTED;
  if (d->causal != 0 && d->causal != 1) return LARD_ERR_INVALID_ARGUMENT;
  if (!(d->scale > 0.0f) || !isfinite(d->scale)) return LARD_ERR_INVALID_ARGUMENT;
  if (d->H < 1) return LARD_ERR_INVALID_ARGUMENT;
  if (d->H > LARD_MAX_HEADS) return LARD_ERR_UNSUPPORTED;
  lard_status s = check_strides(d->dtype, d->t_stride_b, d->t_stride_h, d->t_stride_n);
  if (s != LARD_OK) return s;
  s = check_strides(d->dtype, d->s_stride_b, d->s_stride_h, d->s_stride_n);
  if (s != LARD_OK) return s;
  // rows must not overlap inside one head (stride over n at least one row of d)
  if (d->N > 1 && (d->t_stride_n < d->d || d->s_stride_n < d->d)) return LARD_ERR_INVALID_ARGUMENT;
  if (d->head_map == nullptr) {
    if (d->H != d->H_in) return LARD_ERR_INVALID_ARGUMENT;
  } else {
    bool seen[LARD_MAX_HEADS * 4];
    if (d->H_in > LARD_MAX_HEADS * 4) return LARD_ERR_UNSUPPORTED;
    memset(seen, 0, sizeof(seen));
    for (int h = 0; h < d->H; ++h) {
      const int32_t v = d->head_map[h];
      if (v < 0 || v >= d->H_in) return LARD_ERR_INVALID_ARGUMENT;
      if (seen[v]) return LARD_ERR_INVALID_ARGUMENT;
      seen[v] = true;
    }
  }
  // 32-bit work indices
  const int64_t units = (int64_t)d->B * d->H;
  const int64_t row_tiles = (d->N + kBR - 1) / kBR;
  if (units * row_tiles * kMaxSplits > 0x7fffffffLL) return LARD_ERR_UNSUPPORTED;
  if ((int64_t)units * d->N > 0x7fffffffLL * 4LL) return LARD_ERR_UNSUPPORTED;
  return LARD_OK;
}

void fill_map(UnitMap& m, const lard_relkl_desc* d) {
  for (int h = 0; h < d->H; ++h) m.head_map[h] = d->head_map ? d->head_map[h] : h;
  for (int h = d->H; h < LARD_MAX_HEADS; ++h) m.head_map[h] = 0;
}

int row_tiles_of(const lard_relkl_desc* d) { return (d->N + kBR - 1) / kBR; }
int bwd_row_tiles_of(const lard_relkl_desc* d) { return (d->N + kBRB - 1) / kBRB; }
int key_tiles_of(const lard_relkl_desc* d) { return (d->N + kBC - 1) / kBC; }

// Split the key range of the backward when the (unit, row tile) grid alone cannot fill
// the chip.  Deterministic in the shape; LARD_SPLITK overrides it (clamped).
int choose_splits(const lard_relkl_desc* d) {
  const int64_t base = (int64_t)d->B * d->H * bwd_row_tiles_of(d);
  const int kt = key_tiles_of(d);
  int s = 1;
  if (base < kTargetWorkgroups) s = (int)((kTargetWorkgroups + base - 1) / base);
  const char* env = getenv("LARD_SPLITK");
  if (env && env[0]) {
    const int v = atoi(env);
    if (v >= 1) s = v;
  }
  if (s > kt) s = kt;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return s;
}

size_t fwd_workspace(const lard_relkl_desc* d) {
  const size_t n = (size_t)d->B * d->H * row_tiles_of(d);
  return ((n * sizeof(double) + 255) / 256) * 256;
}

ReserveLayout reserve_of(const lard_relkl_desc* d) {
  return reserve_layout((int64_t)d->B * d->H, d->N, d->d, d->dtype == LARD_BF16 ? 2 : 0);
}

// RoPE-fused entry points: rotated copies of both sides, fp16 (bf16 inputs) or fp32.
ReserveLayout rope_reserve_of(const lard_relkl_desc* d) {
  return reserve_layout((int64_t)d->B * d->H, d->N, d->d, d->dtype == LARD_BF16 ? 2 : 4);
}

// Tables of one side: both null (not rotated) or both set, 16-byte aligned.
lard_status check_tables(const float* c, const float* s) {
  if ((c == nullptr) != (s == nullptr)) return LARD_ERR_INVALID_ARGUMENT;
  if (c && (!aligned(c, 16) || !aligned(s, 16))) return LARD_ERR_INVALID_ARGUMENT;
  return LARD_OK;
}

lard_status check_rope(const lard_rope_desc* r) {
  if (!r) return LARD_ERR_INVALID_ARGUMENT;
  const lard_status s = check_tables(r->cos_teacher, r->sin_teacher);
  if (s != LARD_OK) return s;
  return check_tables(r->cos_student, r->sin_student);
}

// Cross relation: rows of A_t, A_s, B_t, B_s copied (rotated when tables are given).
ReserveLayout cross_reserve_of(const lard_relkl_desc* d) {
  return reserve_layout((int64_t)d->B * d->H, d->N, d->d, d->dtype == LARD_BF16 ? 2 : 4, true);
}

lard_status check_cross(const lard_relkl_desc* d, const lard_cross_desc* k) {
  if (!k) return LARD_ERR_INVALID_ARGUMENT;
  lard_status s = check_strides(d->dtype, k->bt_stride_b, k->bt_stride_h, k->bt_stride_n);
  if (s != LARD_OK) return s;
  s = check_strides(d->dtype, k->bs_stride_b, k->bs_stride_h, k->bs_stride_n);
  if (s != LARD_OK) return s;
  if (d->N > 1 && (k->bt_stride_n < d->d || k->bs_stride_n < d->d)) return LARD_ERR_INVALID_ARGUMENT;
  return LARD_OK;
}

lard_status check_grad(const lard_relkl_desc* desc, const lard_grad_desc* grad, const void* dx) {
  if (!grad || !dx) return LARD_ERR_INVALID_ARGUMENT;
  if (grad->dtype != LARD_FP32 && grad->dtype != LARD_BF16) return LARD_ERR_INVALID_ARGUMENT;
  if (grad->dtype == LARD_BF16 && desc->dtype != LARD_BF16) return LARD_ERR_UNSUPPORTED;
  const lard_status s = check_strides(grad->dtype, grad->stride_b, grad->stride_h, grad->stride_n);
  if (s != LARD_OK) return s;
  if (desc->N > 1 && grad->stride_n < desc->d) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(dx, 16)) return LARD_ERR_INVALID_ARGUMENT;
  return LARD_OK;
}

// Backward launch plus the split-K reduction, writing one gradient.
lard_status run_bwd(const lard_relkl_desc* desc, BwdArgs& a, const lard_grad_desc* grad,
                    void* dx, int mode, void* stream) {
  a.g_sb = grad->stride_b; a.g_sh = grad->stride_h; a.g_sn = grad->stride_n;
  a.dx = dx;
  const bool out_f32 = grad->dtype == LARD_FP32;
  int e = launch_bwd(a, desc->dtype == LARD_BF16, desc->d, desc->causal == 1, out_f32, stream,
                     mode);
  if (e != 0) return LARD_ERR_HIP;
  if (a.splits > 1) {
    ReduceArgs r;
    memset(&r, 0, sizeof(r));
    r.partial = a.partial;
    r.dx = dx;
    r.g_sb = a.g_sb; r.g_sh = a.g_sh; r.g_sn = a.g_sn;
    r.B = a.B; r.H = a.H; r.N = a.N; r.d = desc->d;
    r.rows_pad = a.row_tiles * kBRB;
    r.splits = a.splits;
    r.map = a.map;
    e = launch_splitk_reduce(r, out_f32, stream);
    if (e != 0) return LARD_ERR_HIP;
  }
  return LARD_OK;
}

size_t bwd_workspace(const lard_relkl_desc* d) {
  const int s = choose_splits(d);
  if (s == 1) return 0;
  return (size_t)s * d->B * d->H * (size_t)bwd_row_tiles_of(d) * kBRB * d->d * sizeof(float);
}

}  // namespace

extern "C" {

const char* lard_status_string(lard_status status) {
  switch (status) {
    case LARD_OK: return "LARD_OK: success";
    case LARD_ERR_INVALID_ARGUMENT: return "LARD_ERR_INVALID_ARGUMENT: invalid argument";
    case LARD_ERR_UNSUPPORTED: return "LARD_ERR_UNSUPPORTED: unsupported configuration";
    case LARD_ERR_WORKSPACE_TOO_SMALL: return "LARD_ERR_WORKSPACE_TOO_SMALL: workspace too small";
    case LARD_ERR_HIP: return "LARD_ERR_HIP: HIP launch or runtime error";
  }
  return "unknown lard_status";
}

int lard_version(void) { return kVersion; }

size_t lard_relkl_workspace_size(const lard_relkl_desc* desc, int pass, lard_status* status) {
  lard_status s = check_desc(desc);
  if (s == LARD_OK && pass != 0 && pass != 1) s = LARD_ERR_INVALID_ARGUMENT;
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return pass == 0 ? fwd_workspace(desc) : bwd_workspace(desc);
}

size_t lard_relkl_reserve_size(const lard_relkl_desc* desc, lard_status* status) {
  const lard_status s = check_desc(desc);
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return reserve_of(desc).total;
}

lard_status lard_relkl_fwd(const lard_relkl_desc* desc, const void* x_teacher,
                           const void* x_student, float* lse_teacher, float* lse_student,
                           float* row_kl, float* loss, void* reserve, size_t reserve_bytes,
                           void* workspace, size_t workspace_bytes, void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if (!x_teacher || !x_student || !lse_teacher || !lse_student || !loss || !workspace ||
      !reserve)
    return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(x_teacher, 16) || !aligned(x_student, 16) || !aligned(workspace, 8) ||
      !aligned(reserve, 256) || !aligned(lse_teacher, 4) || !aligned(lse_student, 4) ||
      !aligned(loss, 4) || (row_kl && !aligned(row_kl, 4)))
    return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fwd_workspace(desc)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const ReserveLayout R = reserve_of(desc);
  if (reserve_bytes < R.total) return LARD_ERR_WORKSPACE_TOO_SMALL;

  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.x_t = x_teacher;
  a.x_s = x_student;
  a.t_sb = desc->t_stride_b; a.t_sh = desc->t_stride_h; a.t_sn = desc->t_stride_n;
  a.s_sb = desc->s_stride_b; a.s_sh = desc->s_stride_h; a.s_sn = desc->s_stride_n;
  a.B = desc->B; a.H = desc->H; a.N = desc->N;
  a.row_tiles = row_tiles_of(desc);
  a.scale = desc->scale;
  a.c2 = desc->scale * 1.4426950408889634f;
  a.lse_t = lse_teacher;
  a.lse_s = lse_student;
  a.row_kl = row_kl;
  a.partial = static_cast<double*>(workspace);
  char* rb = static_cast<char*>(reserve);
  a.npad = (int32_t)R.npad;
  a.x16_t = desc->dtype == LARD_BF16 ? reinterpret_cast<uint16_t*>(rb + R.x16_t) : nullptr;
  a.x16_s = desc->dtype == LARD_BF16 ? reinterpret_cast<uint16_t*>(rb + R.x16_s) : nullptr;
  a.r_t = reinterpret_cast<float*>(rb + R.r_t);
  a.r_s = reinterpret_cast<float*>(rb + R.r_s);
  fill_map(a.map, desc);
  const int e = launch_fwd(a, desc->dtype == LARD_BF16, desc->d, desc->causal == 1, loss, stream);
  return e == 0 ? LARD_OK : LARD_ERR_HIP;
}

lard_status lard_relkl_bwd(const lard_relkl_desc* desc, const void* x_teacher,
                           const void* x_student, const void* reserve, size_t reserve_bytes,
                           const float* grad_loss, const lard_grad_desc* grad,
                           void* dx_student, void* workspace, size_t workspace_bytes,
                           void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if (!grad || !x_teacher || !x_student || !reserve || !grad_loss || !dx_student)
    return LARD_ERR_INVALID_ARGUMENT;
  if (grad->dtype != LARD_FP32 && grad->dtype != LARD_BF16) return LARD_ERR_INVALID_ARGUMENT;
  if (grad->dtype == LARD_BF16 && desc->dtype != LARD_BF16) return LARD_ERR_UNSUPPORTED;
  s = check_strides(grad->dtype, grad->stride_b, grad->stride_h, grad->stride_n);
  if (s != LARD_OK) return s;
  if (desc->N > 1 && grad->stride_n < desc->d) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(x_teacher, 16) || !aligned(x_student, 16) || !aligned(dx_student, 16) ||
      !aligned(reserve, 256) || !aligned(grad_loss, 4))
    return LARD_ERR_INVALID_ARGUMENT;
  const ReserveLayout R = reserve_of(desc);
  if (reserve_bytes < R.total) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const size_t need = bwd_workspace(desc);
  if (need > 0 && (!workspace || !aligned(workspace, 16))) return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return LARD_ERR_WORKSPACE_TOO_SMALL;

  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.x_t = x_teacher;
  a.x_s = x_student;
  a.t_sb = desc->t_stride_b; a.t_sh = desc->t_stride_h; a.t_sn = desc->t_stride_n;
  a.s_sb = desc->s_stride_b; a.s_sh = desc->s_stride_h; a.s_sn = desc->s_stride_n;
  a.g_sb = grad->stride_b; a.g_sh = grad->stride_h; a.g_sn = grad->stride_n;
  a.B = desc->B; a.H = desc->H; a.N = desc->N;
  a.row_tiles = bwd_row_tiles_of(desc);
  a.key_tiles = key_tiles_of(desc);
  a.splits = choose_splits(desc);
  a.scale = desc->scale;
  a.c2 = desc->scale * 1.4426950408889634f;
  const char* rb = static_cast<const char*>(reserve);
  a.npad = (int32_t)R.npad;
  a.x16_t = desc->dtype == LARD_BF16 ? reinterpret_cast<const uint16_t*>(rb + R.x16_t) : nullptr;
  a.x16_s = desc->dtype == LARD_BF16 ? reinterpret_cast<const uint16_t*>(rb + R.x16_s) : nullptr;
  a.y16_t = a.x16_t;
  a.y16_s = a.x16_s;
  a.r_t = reinterpret_cast<const float*>(rb + R.r_t);
  a.r_s = reinterpret_cast<const float*>(rb + R.r_s);
  a.rc_t = a.r_t;
  a.rc_s = a.r_s;
  a.grad_loss = grad_loss;
  a.dx = dx_student;
  a.partial = static_cast<float*>(workspace);
  fill_map(a.map, desc);
  const bool out_f32 = grad->dtype == LARD_FP32;
  int e = launch_bwd(a, desc->dtype == LARD_BF16, desc->d, desc->causal == 1, out_f32, stream);
  if (e != 0) return LARD_ERR_HIP;
  if (a.splits > 1) {
    ReduceArgs r;
    memset(&r, 0, sizeof(r));
    r.partial = a.partial;
    r.dx = dx_student;
    r.g_sb = a.g_sb; r.g_sh = a.g_sh; r.g_sn = a.g_sn;
    r.B = a.B; r.H = a.H; r.N = a.N; r.d = desc->d;
    r.rows_pad = a.row_tiles * kBRB;
    r.splits = a.splits;
    r.map = a.map;
    e = launch_splitk_reduce(r, out_f32, stream);
    if (e != 0) return LARD_ERR_HIP;
  }
  return LARD_OK;
}

size_t lard_relkl_rope_reserve_size(const lard_relkl_desc* desc, lard_status* status) {
  const lard_status s = check_desc(desc);
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return rope_reserve_of(desc).total;
}

lard_status lard_relkl_rope_fwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                const void* x_teacher, const void* x_student,
                                float* lse_teacher, float* lse_student, float* row_kl,
                                float* loss, void* reserve, size_t reserve_bytes,
                                void* workspace, size_t workspace_bytes, void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  s = check_rope(rope);
  if (s != LARD_OK) return s;
  if (!x_teacher || !x_student || !lse_teacher || !lse_student || !loss || !workspace ||
      !reserve)
    return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(x_teacher, 16) || !aligned(x_student, 16) || !aligned(workspace, 8) ||
      !aligned(reserve, 256) || !aligned(lse_teacher, 4) || !aligned(lse_student, 4) ||
      !aligned(loss, 4) || (row_kl && !aligned(row_kl, 4)))
    return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fwd_workspace(desc)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const ReserveLayout R = rope_reserve_of(desc);
  if (reserve_bytes < R.total) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const bool bf16 = desc->dtype == LARD_BF16;
  char* rb = static_cast<char*>(reserve);

  // 1. rotated copies of both sides into the reserve
  PrepArgs p;
  memset(&p, 0, sizeof(p));
  p.x_t = x_teacher;
  p.x_s = x_student;
  p.t_sb = desc->t_stride_b; p.t_sh = desc->t_stride_h; p.t_sn = desc->t_stride_n;
  p.s_sb = desc->s_stride_b; p.s_sh = desc->s_stride_h; p.s_sn = desc->s_stride_n;
  p.B = desc->B; p.H = desc->H; p.N = desc->N;
  p.cos_t = rope->cos_teacher; p.sin_t = rope->sin_teacher;
  p.cos_s = rope->cos_student; p.sin_s = rope->sin_student;
  p.c_t = rb + R.x16_t;
  p.c_s = rb + R.x16_s;
  fill_map(p.map, desc);
  int e = launch_rope_prep(p, bf16, desc->d, stream);
  if (e != 0) return LARD_ERR_HIP;

  // 2. the forward on the copies: dense [unit][N][d], read through the identity map
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.x_t = rb + R.x16_t;
  a.x_s = rb + R.x16_s;
  const int64_t sn = desc->d, sh = (int64_t)desc->N * desc->d, sb = (int64_t)desc->H * sh;
  a.t_sb = sb; a.t_sh = sh; a.t_sn = sn;
  a.s_sb = sb; a.s_sh = sh; a.s_sn = sn;
  a.B = desc->B; a.H = desc->H; a.N = desc->N;
  a.row_tiles = row_tiles_of(desc);
  a.scale = desc->scale;
  a.c2 = desc->scale * 1.4426950408889634f;
  a.lse_t = lse_teacher;
  a.lse_s = lse_student;
  a.row_kl = row_kl;
  a.partial = static_cast<double*>(workspace);
  a.npad = (int32_t)R.npad;
  a.r_t = reinterpret_cast<float*>(rb + R.r_t);
  a.r_s = reinterpret_cast<float*>(rb + R.r_s);
  for (int h = 0; h < LARD_MAX_HEADS; ++h) a.map.head_map[h] = h < desc->H ? h : 0;
  e = launch_fwd(a, bf16, desc->d, desc->causal == 1, loss, stream, /*f16_copies=*/bf16);
  return e == 0 ? LARD_OK : LARD_ERR_HIP;
}

lard_status lard_relkl_rope_bwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                const void* reserve, size_t reserve_bytes,
                                const float* grad_loss, const lard_grad_desc* grad,
                                void* dx_student, void* workspace, size_t workspace_bytes,
                                void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  s = check_rope(rope);
  if (s != LARD_OK) return s;
  if (!grad || !reserve || !grad_loss || !dx_student) return LARD_ERR_INVALID_ARGUMENT;
  if (grad->dtype != LARD_FP32 && grad->dtype != LARD_BF16) return LARD_ERR_INVALID_ARGUMENT;
  if (grad->dtype == LARD_BF16 && desc->dtype != LARD_BF16) return LARD_ERR_UNSUPPORTED;
  s = check_strides(grad->dtype, grad->stride_b, grad->stride_h, grad->stride_n);
  if (s != LARD_OK) return s;
  if (desc->N > 1 && grad->stride_n < desc->d) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(dx_student, 16) || !aligned(reserve, 256) || !aligned(grad_loss, 4))
    return LARD_ERR_INVALID_ARGUMENT;
  const ReserveLayout R = rope_reserve_of(desc);
  if (reserve_bytes < R.total) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const size_t need = bwd_workspace(desc);
  if (need > 0 && (!workspace || !aligned(workspace, 16))) return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const bool bf16 = desc->dtype == LARD_BF16;
  const char* rb = static_cast<const char*>(reserve);

  BwdArgs a;
  memset(&a, 0, sizeof(a));
  // operands: the rotated copies (fp16 through x16_*, fp32 through x_* read densely)
  a.x_t = rb + R.x16_t;
  a.x_s = rb + R.x16_s;
  a.y_t = a.x_t;
  a.y_s = a.x_s;
  a.x_unit_dense = 1;
  a.g_sb = grad->stride_b; a.g_sh = grad->stride_h; a.g_sn = grad->stride_n;
  a.B = desc->B; a.H = desc->H; a.N = desc->N;
  a.row_tiles = bwd_row_tiles_of(desc);
  a.key_tiles = key_tiles_of(desc);
  a.splits = choose_splits(desc);
  a.scale = desc->scale;
  a.c2 = desc->scale * 1.4426950408889634f;
  a.npad = (int32_t)R.npad;
  a.x16_t = bf16 ? reinterpret_cast<const uint16_t*>(rb + R.x16_t) : nullptr;
  a.x16_s = bf16 ? reinterpret_cast<const uint16_t*>(rb + R.x16_s) : nullptr;
  a.y16_t = a.x16_t;
  a.y16_s = a.x16_s;
  a.r_t = reinterpret_cast<const float*>(rb + R.r_t);
  a.r_s = reinterpret_cast<const float*>(rb + R.r_s);
  a.rc_t = a.r_t;
  a.rc_s = a.r_s;
  a.grad_loss = grad_loss;
  a.rope_cos = rope->cos_student;
  a.rope_sin = rope->sin_student;
  a.dx = dx_student;
  a.partial = static_cast<float*>(workspace);
  fill_map(a.map, desc);  // output placement only: operands are read per unit
  const bool out_f32 = grad->dtype == LARD_FP32;
  int e = launch_bwd(a, bf16, desc->d, desc->causal == 1, out_f32, stream);
  if (e != 0) return LARD_ERR_HIP;
  if (a.splits > 1) {
    ReduceArgs r;
    memset(&r, 0, sizeof(r));
    r.partial = a.partial;
    r.dx = dx_student;
    r.g_sb = a.g_sb; r.g_sh = a.g_sh; r.g_sn = a.g_sn;
    r.B = a.B; r.H = a.H; r.N = a.N; r.d = desc->d;
    r.rows_pad = a.row_tiles * kBRB;
    r.splits = a.splits;
    r.map = a.map;
    e = launch_splitk_reduce(r, out_f32, stream);
    if (e != 0) return LARD_ERR_HIP;
  }
  return LARD_OK;
}

size_t lard_relkl_cross_reserve_size(const lard_relkl_desc* desc, lard_status* status) {
  const lard_status s = check_desc(desc);
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return cross_reserve_of(desc).total;
}

lard_status lard_relkl_cross_fwd(const lard_relkl_desc* desc, const lard_cross_desc* keys,
                                 const lard_rope_desc* rope, const void* a_teacher,
                                 const void* b_teacher, const void* a_student,
                                 const void* b_student, float* lse_teacher, float* lse_student,
                                 float* row_kl, float* loss, void* reserve, size_t reserve_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  s = check_cross(desc, keys);
  if (s != LARD_OK) return s;
  if (rope) {
    s = check_rope(rope);
    if (s != LARD_OK) return s;
  }
  if (!a_teacher || !b_teacher || !a_student || !b_student || !lse_teacher || !lse_student ||
      !loss || !workspace || !reserve)
    return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(a_teacher, 16) || !aligned(b_teacher, 16) || !aligned(a_student, 16) ||
      !aligned(b_student, 16) || !aligned(workspace, 8) || !aligned(reserve, 256) ||
      !aligned(lse_teacher, 4) || !aligned(lse_student, 4) || !aligned(loss, 4) ||
      (row_kl && !aligned(row_kl, 4)))
    return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fwd_workspace(desc)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const ReserveLayout R = cross_reserve_of(desc);
  if (reserve_bytes < R.total) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const bool bf16 = desc->dtype == LARD_BF16;
  char* rb = static_cast<char*>(reserve);

  // 1. copies (rotated when tables are given) of A and B of both sides
  for (int side = 0; side < 2; ++side) {
    PrepArgs p;
    memset(&p, 0, sizeof(p));
    p.B = desc->B; p.H = desc->H; p.N = desc->N;
    if (rope) {
      p.cos_t = rope->cos_teacher; p.sin_t = rope->sin_teacher;
      p.cos_s = rope->cos_student; p.sin_s = rope->sin_student;
    }
    fill_map(p.map, desc);
    if (side == 0) {
      p.x_t = a_teacher;
      p.x_s = a_student;
      p.t_sb = desc->t_stride_b; p.t_sh = desc->t_stride_h; p.t_sn = desc->t_stride_n;
      p.s_sb = desc->s_stride_b; p.s_sh = desc->s_stride_h; p.s_sn = desc->s_stride_n;
      p.c_t = rb + R.x16_t;
      p.c_s = rb + R.x16_s;
    } else {
      p.x_t = b_teacher;
      p.x_s = b_student;
      p.t_sb = keys->bt_stride_b; p.t_sh = keys->bt_stride_h; p.t_sn = keys->bt_stride_n;
      p.s_sb = keys->bs_stride_b; p.s_sh = keys->bs_stride_h; p.s_sn = keys->bs_stride_n;
      p.c_t = rb + R.y16_t;
      p.c_s = rb + R.y16_s;
    }
    if (launch_rope_prep(p, bf16, desc->d, stream) != 0) return LARD_ERR_HIP;
  }

  // 2. the forward: own rows from the A copies, key tiles from the B copies
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.x_t = rb + R.x16_t;
  a.x_s = rb + R.x16_s;
  a.y_t = rb + R.y16_t;
  a.y_s = rb + R.y16_s;
  const int64_t sn = desc->d, sh = (int64_t)desc->N * desc->d, sb = (int64_t)desc->H * sh;
  a.t_sb = sb; a.t_sh = sh; a.t_sn = sn;
  a.s_sb = sb; a.s_sh = sh; a.s_sn = sn;
  a.B = desc->B; a.H = desc->H; a.N = desc->N;
  a.row_tiles = row_tiles_of(desc);
  a.scale = desc->scale;
  a.c2 = desc->scale * 1.4426950408889634f;
  a.lse_t = lse_teacher;
  a.lse_s = lse_student;
  a.row_kl = row_kl;
  a.partial = static_cast<double*>(workspace);
  a.npad = (int32_t)R.npad;
  a.r_t = reinterpret_cast<float*>(rb + R.r_t);
  a.r_s = reinterpret_cast<float*>(rb + R.r_s);
  for (int h = 0; h < LARD_MAX_HEADS; ++h) a.map.head_map[h] = h < desc->H ? h : 0;
  const int e = launch_fwd(a, bf16, desc->d, desc->causal == 1, loss, stream, /*f16_copies=*/bf16);
  return e == 0 ? LARD_OK : LARD_ERR_HIP;
}

lard_status lard_relkl_cross_bwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                 const void* reserve, size_t reserve_bytes,
                                 const float* grad_loss, const lard_grad_desc* grad_a,
                                 void* da_student, const lard_grad_desc* grad_b,
                                 void* db_student, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if (rope) {
    s = check_rope(rope);
    if (s != LARD_OK) return s;
  }
  if (!reserve || !grad_loss) return LARD_ERR_INVALID_ARGUMENT;
  s = check_grad(desc, grad_a, da_student);
  if (s != LARD_OK) return s;
  s = check_grad(desc, grad_b, db_student);
  if (s != LARD_OK) return s;
  if (!aligned(reserve, 256) || !aligned(grad_loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
  const ReserveLayout R = cross_reserve_of(desc);
  if (reserve_bytes < R.total) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const size_t need = bwd_workspace(desc);
  if (need > 0 && (!workspace || !aligned(workspace, 16))) return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const bool bf16 = desc->dtype == LARD_BF16;
  const char* rb = static_cast<const char*>(reserve);

  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.x_unit_dense = 1;
  a.B = desc->B; a.H = desc->H; a.N = desc->N;
  a.row_tiles = bwd_row_tiles_of(desc);
  a.key_tiles = key_tiles_of(desc);
  a.splits = choose_splits(desc);
  a.scale = desc->scale;
  a.c2 = desc->scale * 1.4426950408889634f;
  a.npad = (int32_t)R.npad;
  a.grad_loss = grad_loss;
  a.partial = static_cast<float*>(workspace);
  if (rope) {
    a.rope_cos = rope->cos_student;
    a.rope_sin = rope->sin_student;
  }
  fill_map(a.map, desc);  // output placement only: operands are read per unit
  const float* qs_t = reinterpret_cast<const float*>(rb + R.r_t);  // query-row statistics
  const float* qs_s = reinterpret_cast<const float*>(rb + R.r_s);
  auto set_operands = [&](size_t own_t, size_t own_s, size_t stg_t, size_t stg_s) {
    a.x_t = rb + own_t;
    a.x_s = rb + own_s;
    a.y_t = rb + stg_t;
    a.y_s = rb + stg_s;
    a.x16_t = bf16 ? reinterpret_cast<const uint16_t*>(rb + own_t) : nullptr;
    a.x16_s = bf16 ? reinterpret_cast<const uint16_t*>(rb + own_s) : nullptr;
    a.y16_t = bf16 ? reinterpret_cast<const uint16_t*>(rb + stg_t) : nullptr;
    a.y16_s = bf16 ? reinterpret_cast<const uint16_t*>(rb + stg_s) : nullptr;
    a.r_t = qs_t; a.r_s = qs_s;
    a.rc_t = qs_t; a.rc_s = qs_s;
  };
  // dA: own rows of A, staged rows of B, row terms
  set_operands(R.x16_t, R.x16_s, R.y16_t, R.y16_s);
  s = run_bwd(desc, a, grad_a, da_student, 1, stream);
  if (s != LARD_OK) return s;
  // dB: own rows of B, staged rows of A with their statistics, column terms
  set_operands(R.y16_t, R.y16_s, R.x16_t, R.x16_s);
  return run_bwd(desc, a, grad_b, db_student, 2, stream);
}

}  // extern "C"
