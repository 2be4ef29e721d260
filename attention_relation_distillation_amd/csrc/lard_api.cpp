// C ABI of the relation-KL library: host-side validation, workspace sizing and launch
// configuration.  Every check runs before the first HIP call, so an invalid request never
// touches the device.  The operation itself is documented in include/lard.h.
//
// Every entry point assembles "launches" (relkl_internal.h): one kernel launch covers one
// or, for the grouped entry points, up to LARD_MAX_GROUP relation problems ("members").
// The single-problem entry points are groups of one.

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "lard.h"
#include "probe_internal.h"
#include "relkl_internal.h"

namespace {

using namespace lard;

constexpr int kVersion = 2 * 10000 + 0 * 100 + 0;
constexpr int kTargetWorkgroups = 512;  // two rounds of one backward workgroup per CU
constexpr int kMaxSplits = 64;
constexpr float kLog2e = 1.4426950408889634f;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

int elem_size(int dtype) { return dtype == LARD_BF16 ? 2 : 4; }

lard_status check_strides(int dtype, int64_t sb, int64_t sh, int64_t sn) {
  const int64_t q = 16 / elem_size(dtype);
  if (sb < 0 || sh < 0 || sn < 0) return LARD_ERR_INVALID_ARGUMENT;
  if (sb % q || sh % q || sn % q) return LARD_ERR_INVALID_ARGUMENT;
  return LARD_OK;
}

// Row strides (elements) whose byte size stays below 2^24.
bool row_stride_ok(int dtype, int64_t sn) { return sn * elem_size(dtype) < (int64_t(1) << 24); }

lard_status check_desc(const lard_relkl_desc* d) {
  if (!d) return LARD_ERR_INVALID_ARGUMENT;
  if (d->dtype != LARD_FP32 && d->dtype != LARD_BF16) return LARD_ERR_INVALID_ARGUMENT;
  if (d->B < 1 || d->H_in < 1 || d->N < 1 || d->d < 1) return LARD_ERR_INVALID_ARGUMENT;
  if (d->d != 64 && d->d != 128) return LARD_ERR_UNSUPPORTED;
  // row and key indices are 32-bit in the kernels, with a tile's width added to them
  if (d->N > LARD_MAX_N) return LARD_ERR_UNSUPPORTED;
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
  // the backward addresses the rows of a key tile as 24-bit offsets from the tile's first row
  if (d->N > 1 && (!row_stride_ok(d->dtype, d->t_stride_n) || !row_stride_ok(d->dtype, d->s_stride_n)))
    return LARD_ERR_UNSUPPORTED;
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
  const int64_t row_tiles = ((int64_t)d->N + kBR - 1) / kBR;
  if (units * row_tiles * kMaxSplits > 0x7fffffffLL) return LARD_ERR_UNSUPPORTED;
  if ((int64_t)units * d->N > 0x7fffffffLL * 4LL) return LARD_ERR_UNSUPPORTED;
  return LARD_OK;
}

int row_tiles_of(const lard_relkl_desc* d) { return (int)(((int64_t)d->N + kBR - 1) / kBR); }
int bwd_rows_of(const lard_relkl_desc* d) { return bwd_rows(d->dtype == LARD_FP32); }
int bwd_row_tiles_of(const lard_relkl_desc* d) {
  return (int)(((int64_t)d->N + bwd_rows_of(d) - 1) / bwd_rows_of(d));
}
int key_tiles_of(const lard_relkl_desc* d) { return (int)(((int64_t)d->N + kBC - 1) / kBC); }
int64_t units_of(const lard_relkl_desc* d) { return (int64_t)d->B * d->H; }

// Split the key range of the backward when the (unit, row tile) workgroups of a launch
// alone cannot fill the chip.  Deterministic in the shapes; LARD_SPLITK overrides it
// (clamped to the largest member's key tiles: a split with no key tile of a smaller
// member writes zero partials).
int choose_splits(int n, const lard_relkl_desc* const* d) {
  int64_t base = 0;
  int kt = 1;
  for (int k = 0; k < n; ++k) {
    base += units_of(d[k]) * bwd_row_tiles_of(d[k]);
    if (key_tiles_of(d[k]) > kt) kt = key_tiles_of(d[k]);
  }
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

// Forward: one fp64 loss partial per workgroup.
int64_t fwd_partials(const lard_relkl_desc* d) { return units_of(d) * row_tiles_of(d); }

size_t fwd_workspace(int n, const lard_relkl_desc* const* d) {
  int64_t p = 0;
  for (int k = 0; k < n; ++k) p += fwd_partials(d[k]);
  return round256((size_t)p * sizeof(double));
}

// Backward workspace: fp32 split-K partials [splits][units][row_tiles * rows][d] per member
// when the key range is split, else nothing.
size_t bwd_partial_floats(const lard_relkl_desc* d) {
  return (size_t)units_of(d) * bwd_row_tiles_of(d) * bwd_rows_of(d) * d->d;
}

size_t bwd_workspace(int n, const lard_relkl_desc* const* d) {
  const int s = choose_splits(n, d);
  if (s == 1) return 0;
  size_t f = 0;
  for (int k = 0; k < n; ++k) f += bwd_partial_floats(d[k]);
  return (size_t)s * f * sizeof(float);
}

// Reserve of one problem: none (plain), rotated copies in the input dtype (RoPE-fused), or
// copies of A and B as fp16 images of bf16 values or fp32 (cross).
enum class Path { kPlain, kRope, kCross };

size_t reserve_total(const lard_relkl_desc* d, Path p) {
  if (p == Path::kPlain) return 0;
  return reserve_layout(units_of(d), d->N, d->d, elem_size(d->dtype), p == Path::kCross).total;
}

ReserveLayout reserve_of(const lard_relkl_desc* d, Path p) {
  return reserve_layout(units_of(d), d->N, d->d, elem_size(d->dtype), p == Path::kCross);
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

// Forward outputs of one problem (diag_delta and row_kl are optional).
lard_status check_fwd_outputs(const float* lse_t, const float* lse_s, const float* diag_delta,
                              const float* row_kl) {
  if (!lse_t || !lse_s) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(lse_t, 4) || !aligned(lse_s, 4) || (row_kl && !aligned(row_kl, 4)) ||
      (diag_delta && !aligned(diag_delta, 4)))
    return LARD_ERR_INVALID_ARGUMENT;
  return LARD_OK;
}

// Forward state the backward reads (diag_delta: the relation only).
lard_status check_bwd_state(const float* lse_t, const float* lse_s, const float* diag_delta,
                            bool relation) {
  if (!lse_t || !lse_s || (relation && !diag_delta)) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(lse_t, 4) || !aligned(lse_s, 4) || (diag_delta && !aligned(diag_delta, 4)))
    return LARD_ERR_INVALID_ARGUMENT;
  return LARD_OK;
}

lard_status check_inputs(const void* xt, const void* xs) {
  if (!xt || !xs) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(xt, 16) || !aligned(xs, 16)) return LARD_ERR_INVALID_ARGUMENT;
  return LARD_OK;
}

// ------------------------------------------------------------------ launch assembly
// Head maps of the members of one call, in the table every launch of the call carries.
struct MapTable {
  int16_t v[kMapSlots];
  int32_t off[kMaxGroup];
};

// False when the maps do not fit the table.
bool build_maps(MapTable& t, int n, const lard_relkl_desc* const* d) {
  memset(&t, 0, sizeof(t));
  int used = 0;
  for (int k = 0; k < n; ++k) {
    if (!d[k]->head_map) {
      t.off[k] = -1;
      continue;
    }
    if (used + d[k]->H > kMapSlots) return false;
    t.off[k] = used;
    for (int h = 0; h < d[k]->H; ++h) t.v[used + h] = (int16_t)d[k]->head_map[h];
    used += d[k]->H;
  }
  return true;
}

template <class M>
void launch_init(Launch<M>& L) {
  memset(&L, 0, sizeof(L));
}

// Appends a member of `count` workgroups (blocks) to L; returns its arguments.
template <class M>
M& add_member(Launch<M>& L, int count) {
  M& m = L.m[L.n];
  L.end[L.n] = (L.n ? L.end[L.n - 1] : 0) + count;
  ++L.n;
  return m;
}

// Input heads of members read in place go through the call's maps.
template <class M>
void use_maps(Launch<M>& L, const MapTable& t) {
  memcpy(L.head_map, t.v, sizeof(t.v));
  for (int k = 0; k < L.n; ++k) L.m[k].map_off = t.off[k];
}

// Dense [unit][N][d] copies in the reserve are read through the identity.
template <class M>
void identity_maps(Launch<M>& L) {
  for (int k = 0; k < L.n; ++k) L.m[k].map_off = -1;
}

// Forward member: shape and outputs (operands set by the caller).
void fwd_common(FwdArgs& a, const lard_relkl_desc* d, float* lse_t, float* lse_s,
                float* diag_delta, float* row_kl, double* partial) {
  a.B = d->B; a.H = d->H; a.N = d->N;
  a.row_tiles = row_tiles_of(d);
  a.scale = d->scale;
  a.c2 = d->scale * kLog2e;
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  a.row_kl = row_kl;
  a.diag_delta = diag_delta;
  a.partial = partial;
}

// Forward operands read in place from the caller's tensors.
void fwd_inputs(FwdArgs& a, const lard_relkl_desc* d, const void* xt, const void* xs) {
  a.x_t = xt;
  a.x_s = xs;
  a.t_sb = d->t_stride_b; a.t_sh = d->t_stride_h; a.t_sn = d->t_stride_n;
  a.s_sb = d->s_stride_b; a.s_sh = d->s_stride_h; a.s_sn = d->s_stride_n;
}

// Forward operands from dense [unit][N][d] reserve copies; y: key-side copies or null.
void fwd_copies(FwdArgs& a, const lard_relkl_desc* d, const char* xt, const char* xs,
                const char* yt, const char* ys) {
  a.x_t = xt;
  a.x_s = xs;
  a.y_t = yt;
  a.y_s = ys;
  const int64_t sn = d->d, sh = (int64_t)d->N * d->d, sb = (int64_t)d->H * sh;
  a.t_sb = sb; a.t_sh = sh; a.t_sn = sn;
  a.s_sb = sb; a.s_sh = sh; a.s_sn = sn;
}

// Rotation (or plain copy, for a side without tables) of one problem's inputs with the
// given strides into dense reserve copies.
void prep_member(PrepLaunch& P, const lard_relkl_desc* d, const void* xt, int64_t tsb,
                 int64_t tsh, int64_t tsn, const void* xs, int64_t ssb, int64_t ssh,
                 int64_t ssn, const lard_rope_desc* rope, void* ct, void* cs) {
  const int64_t total = 2 * units_of(d) * d->N * (d->d / 8);
  PrepArgs& p = add_member(P, (int)((total + 255) / 256));
  p.x_t = xt;
  p.x_s = xs;
  p.t_sb = tsb; p.t_sh = tsh; p.t_sn = tsn;
  p.s_sb = ssb; p.s_sh = ssh; p.s_sn = ssn;
  p.B = d->B; p.H = d->H; p.N = d->N;
  if (rope) {
    p.cos_t = rope->cos_teacher; p.sin_t = rope->sin_teacher;
    p.cos_s = rope->cos_student; p.sin_s = rope->sin_student;
  }
  p.c_t = ct;
  p.c_s = cs;
}

// Backward member: shape, the forward's state, split and output (operands set by the
// caller).
void bwd_common(BwdArgs& a, const lard_relkl_desc* d, const float* lse_t, const float* lse_s,
                int splits, const float* diag_delta, const float* grad_loss,
                const lard_grad_desc* g, void* dx, float* partial) {
  a.B = d->B; a.H = d->H; a.N = d->N;
  a.row_tiles = bwd_row_tiles_of(d);
  a.key_tiles = key_tiles_of(d);
  a.splits = splits;
  a.scale = d->scale;
  a.c2 = d->scale * kLog2e;
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  a.lc_t = lse_t;
  a.lc_s = lse_s;
  a.diag_delta = diag_delta;
  a.grad_loss = grad_loss;
  a.g_sb = g->stride_b; a.g_sh = g->stride_h; a.g_sn = g->stride_n;
  a.dx = dx;
  a.partial = partial;
}

// Backward operands read in place from the caller's tensors.
void bwd_inputs(BwdArgs& a, const lard_relkl_desc* d, const void* xt, const void* xs) {
  a.x_t = xt;
  a.x_s = xs;
  a.t_sb = d->t_stride_b; a.t_sh = d->t_stride_h; a.t_sn = d->t_stride_n;
  a.s_sb = d->s_stride_b; a.s_sh = d->s_stride_h; a.s_sn = d->s_stride_n;
}

// Backward operands from dense reserve copies (own rows at own_*, staged rows at stg_*).
void bwd_copies(BwdArgs& a, const char* rb, size_t own_t, size_t own_s, size_t stg_t,
                size_t stg_s) {
  a.x_dense = 1;
  a.x_t = rb + own_t;
  a.x_s = rb + own_s;
  a.y_t = rb + stg_t;
  a.y_s = rb + stg_s;
}

int bwd_workgroups(const lard_relkl_desc* d, int splits) {
  return (int)(units_of(d) * bwd_row_tiles_of(d) * splits);
}

// Backward launch plus the split-K reduction of every member.
lard_status run_bwd(const BwdLaunch& L, const lard_relkl_desc* const* d, bool out_f32, int mode,
                    void* stream) {
  const lard_relkl_desc* d0 = d[0];
  int e = launch_bwd(L, d0->dtype == LARD_BF16, d0->d, d0->causal == 1, out_f32, stream, mode);
  if (e != 0) return LARD_ERR_HIP;
  if (L.m[0].splits > 1) {
    ReduceLaunch R;
    launch_init(R);
    for (int k = 0; k < L.n; ++k) {
      const BwdArgs& a = L.m[k];
      const int64_t total = units_of(d[k]) * d[k]->N * (d[k]->d / 4);
      ReduceArgs& r = add_member(R, (int)((total + 255) / 256));
      r.partial = a.partial;
      r.dx = a.dx;
      r.g_sb = a.g_sb; r.g_sh = a.g_sh; r.g_sn = a.g_sn;
      r.B = a.B; r.H = a.H; r.N = a.N; r.d = d[k]->d;
      r.rows_pad = a.row_tiles * bwd_rows_of(d[k]);
      r.splits = a.splits;
      r.map_off = a.map_off;
    }
    memcpy(R.head_map, L.head_map, sizeof(R.head_map));
    e = launch_splitk_reduce(R, out_f32, stream);
    if (e != 0) return LARD_ERR_HIP;
  }
  return LARD_OK;
}

// Loss outputs of a forward launch whose members' partials start at `partial`.
LossOut loss_out(const FwdLaunch& L, double* partial, float* total, float* const* member) {
  LossOut o;
  memset(&o, 0, sizeof(o));
  o.partial = partial;
  o.total = total;
  o.n = L.n;
  for (int k = 0; k < L.n; ++k) {
    o.member[k] = member ? member[k] : nullptr;
    o.begin[k + 1] = L.end[k];
  }
  return o;
}

// ------------------------------------------------------------------ grouped problems
// Common requirements of a group: valid members that share dtype, d and mask, head maps
// that fit one table, 32-bit work indices.
lard_status check_group(int n, const lard_relkl_member* m, const lard_relkl_desc** d) {
  if (n < 1 || !m) return LARD_ERR_INVALID_ARGUMENT;
  if (n > LARD_MAX_GROUP) return LARD_ERR_UNSUPPORTED;
  int64_t work = 0, rows = 0;
  for (int k = 0; k < n; ++k) {
    d[k] = &m[k].desc;
    const lard_status s = check_desc(d[k]);
    if (s != LARD_OK) return s;
    if (d[k]->dtype != d[0]->dtype || d[k]->d != d[0]->d || d[k]->causal != d[0]->causal)
      return LARD_ERR_INVALID_ARGUMENT;
    work += units_of(d[k]) * row_tiles_of(d[k]);
    rows += units_of(d[k]) * d[k]->N;
  }
  // 32-bit grids over all members: workgroups with splits, and the per-row passes
  if (work * kMaxSplits > 0x7fffffffLL) return LARD_ERR_UNSUPPORTED;
  if (rows > 0x7fffffffLL * 4LL) return LARD_ERR_UNSUPPORTED;
  MapTable t;
  if (!build_maps(t, n, d)) return LARD_ERR_UNSUPPORTED;
  return LARD_OK;
}

size_t group_reserve(int n, const lard_relkl_desc* const* d, Path p, size_t* off) {
  size_t total = 0;
  for (int k = 0; k < n; ++k) {
    if (off) off[k] = total;
    total += reserve_total(d[k], p);
  }
  return total;
}

// Forward of n problems (plain or RoPE-fused) with reserve regions at rb + off[k].
lard_status run_group_fwd(int n, const lard_relkl_desc* const* d, const void* const* xt,
                          const void* const* xs, float* const* lse_t, float* const* lse_s,
                          float* const* diag_delta, float* const* row_kl,
                          float* const* member_loss, const lard_rope_desc* const* rope,
                          bool with_rope, float* loss, char* rb, const size_t* off,
                          double* partial, void* stream) {
  const bool bf16 = d[0]->dtype == LARD_BF16;
  MapTable maps;
  build_maps(maps, n, d);
  if (with_rope) {
    // 1. rotated copies of every member into its reserve region, in the input dtype
    PrepLaunch P;
    launch_init(P);
    for (int k = 0; k < n; ++k) {
      const ReserveLayout R = reserve_of(d[k], Path::kRope);
      char* r = rb + off[k];
      prep_member(P, d[k], xt[k], d[k]->t_stride_b, d[k]->t_stride_h, d[k]->t_stride_n, xs[k],
                  d[k]->s_stride_b, d[k]->s_stride_h, d[k]->s_stride_n, rope[k], r + R.x_t,
                  r + R.x_s);
    }
    use_maps(P, maps);
    if (launch_rope_prep(P, bf16, d[0]->d, stream, /*f16_images=*/false) != 0)
      return LARD_ERR_HIP;
  }
  // 2. the forward: in place (plain) or on the copies
  FwdLaunch F;
  launch_init(F);
  double* part = partial;
  for (int k = 0; k < n; ++k) {
    FwdArgs& a = add_member(F, (int)fwd_partials(d[k]));
    if (with_rope) {
      const ReserveLayout R = reserve_of(d[k], Path::kRope);
      fwd_copies(a, d[k], rb + off[k] + R.x_t, rb + off[k] + R.x_s, nullptr, nullptr);
    } else {
      fwd_inputs(a, d[k], xt[k], xs[k]);
    }
    fwd_common(a, d[k], lse_t[k], lse_s[k], diag_delta[k], row_kl[k], part);
    part += fwd_partials(d[k]);
  }
  if (with_rope) identity_maps(F);
  else use_maps(F, maps);
  const LossOut lo = loss_out(F, partial, loss, member_loss);
  const int e = launch_fwd(F, bf16, d[0]->d, d[0]->causal == 1, lo, stream, /*cross=*/false);
  return e == 0 ? LARD_OK : LARD_ERR_HIP;
}

// Backward of n problems (plain or RoPE-fused), one gradient dtype.
lard_status run_group_bwd(int n, const lard_relkl_desc* const* d, const void* const* xt,
                          const void* const* xs, const float* const* lse_t,
                          const float* const* lse_s, const float* const* diag_delta,
                          const lard_rope_desc* const* rope, bool with_rope, const char* rb,
                          const size_t* off, const float* grad_loss,
                          const lard_grad_desc* const* grad, void* const* dx, float* partial,
                          void* stream) {
  const int splits = choose_splits(n, d);
  MapTable maps;
  build_maps(maps, n, d);
  BwdLaunch L;
  launch_init(L);
  float* part = partial;
  for (int k = 0; k < n; ++k) {
    BwdArgs& a = add_member(L, bwd_workgroups(d[k], splits));
    if (with_rope) {
      const ReserveLayout R = reserve_of(d[k], Path::kRope);
      bwd_copies(a, rb + off[k], R.x_t, R.x_s, R.x_t, R.x_s);
      a.rope_cos = rope[k] ? rope[k]->cos_student : nullptr;
      a.rope_sin = rope[k] ? rope[k]->sin_student : nullptr;
    } else {
      bwd_inputs(a, d[k], xt[k], xs[k]);
    }
    bwd_common(a, d[k], lse_t[k], lse_s[k], splits, diag_delta[k], grad_loss, grad[k], dx[k],
               part);
    if (splits > 1) part += (size_t)splits * bwd_partial_floats(d[k]);
  }
  use_maps(L, maps);  // output placement (and in-place operands of the plain path)
  return run_bwd(L, d, grad[0]->dtype == LARD_FP32, 0, stream);
}

// Workspace argument check of a backward needing `need` bytes.
lard_status check_bwd_workspace(const void* ws, size_t bytes, size_t need) {
  if (need > 0 && (!ws || !aligned(ws, 16))) return LARD_ERR_INVALID_ARGUMENT;
  if (bytes < need) return LARD_ERR_WORKSPACE_TOO_SMALL;
  return LARD_OK;
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

lard_status lard_probe_mfma(int vector_work, int iters, int workgroups, float* sink,
                            void* stream) {
  if (!sink || !aligned(sink, 4) || iters < 1 || iters > (1 << 20) || workgroups < 1 ||
      workgroups > (1 << 16) || (vector_work != 0 && vector_work != 1))
    return LARD_ERR_INVALID_ARGUMENT;
  return launch_probe_mfma(vector_work == 1, iters, workgroups, sink, stream) == 0
             ? LARD_OK
             : LARD_ERR_HIP;
}

size_t lard_relkl_workspace_size(const lard_relkl_desc* desc, int pass, lard_status* status) {
  lard_status s = check_desc(desc);
  if (s == LARD_OK && pass != 0 && pass != 1) s = LARD_ERR_INVALID_ARGUMENT;
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return pass == 0 ? fwd_workspace(1, &desc) : bwd_workspace(1, &desc);
}

lard_status lard_relkl_fwd(const lard_relkl_desc* desc, const void* x_teacher,
                           const void* x_student, float* lse_teacher, float* lse_student,
                           float* diag_delta, float* row_kl, float* loss, void* workspace,
                           size_t workspace_bytes, void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if ((s = check_inputs(x_teacher, x_student)) != LARD_OK) return s;
  if ((s = check_fwd_outputs(lse_teacher, lse_student, diag_delta, row_kl)) != LARD_OK) return s;
  if (!loss || !workspace) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 8) || !aligned(loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fwd_workspace(1, &desc)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  return run_group_fwd(1, &desc, &x_teacher, &x_student, &lse_teacher, &lse_student,
                       &diag_delta, &row_kl, nullptr, nullptr, false, loss, nullptr, nullptr,
                       static_cast<double*>(workspace), stream);
}

lard_status lard_relkl_bwd(const lard_relkl_desc* desc, const void* x_teacher,
                           const void* x_student, const float* lse_teacher,
                           const float* lse_student, const float* diag_delta,
                           const float* grad_loss, const lard_grad_desc* grad,
                           void* dx_student, void* workspace, size_t workspace_bytes,
                           void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if ((s = check_inputs(x_teacher, x_student)) != LARD_OK) return s;
  if ((s = check_bwd_state(lse_teacher, lse_student, diag_delta, true)) != LARD_OK) return s;
  if (!grad_loss || !aligned(grad_loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
  if ((s = check_grad(desc, grad, dx_student)) != LARD_OK) return s;
  s = check_bwd_workspace(workspace, workspace_bytes, bwd_workspace(1, &desc));
  if (s != LARD_OK) return s;
  return run_group_bwd(1, &desc, &x_teacher, &x_student, &lse_teacher, &lse_student,
                       &diag_delta, nullptr, false, nullptr, nullptr, grad_loss, &grad,
                       &dx_student, static_cast<float*>(workspace), stream);
}

lard_status lard_relkl_fwd_noalloc(const lard_relkl_desc* desc, const void* x_teacher,
                                   const void* x_student, float* lse_teacher,
                                   float* lse_student, float* diag_delta, float* row_kl,
                                   float* loss, void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if ((s = check_inputs(x_teacher, x_student)) != LARD_OK) return s;
  if ((s = check_fwd_outputs(lse_teacher, lse_student, diag_delta, row_kl)) != LARD_OK) return s;
  if (!loss || !aligned(loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
  if (fwd_partials(desc) > kNoallocMaxPartials) return LARD_ERR_WORKSPACE_TOO_SMALL;
  void* scratch = nullptr;
  if (scratch_address(&scratch) != 0) return LARD_ERR_HIP;
  return run_group_fwd(1, &desc, &x_teacher, &x_student, &lse_teacher, &lse_student,
                       &diag_delta, &row_kl, nullptr, nullptr, false, loss, nullptr, nullptr,
                       static_cast<double*>(scratch), stream);
}

size_t lard_relkl_rope_reserve_size(const lard_relkl_desc* desc, lard_status* status) {
  const lard_status s = check_desc(desc);
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return reserve_total(desc, Path::kRope);
}

lard_status lard_relkl_rope_fwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                const void* x_teacher, const void* x_student,
                                float* lse_teacher, float* lse_student, float* diag_delta,
                                float* row_kl, float* loss, void* reserve, size_t reserve_bytes,
                                void* workspace, size_t workspace_bytes, void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if ((s = check_rope(rope)) != LARD_OK) return s;
  if ((s = check_inputs(x_teacher, x_student)) != LARD_OK) return s;
  if ((s = check_fwd_outputs(lse_teacher, lse_student, diag_delta, row_kl)) != LARD_OK) return s;
  if (!loss || !workspace || !reserve) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 8) || !aligned(reserve, 256) || !aligned(loss, 4))
    return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fwd_workspace(1, &desc)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  if (reserve_bytes < reserve_total(desc, Path::kRope)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const size_t off = 0;
  return run_group_fwd(1, &desc, &x_teacher, &x_student, &lse_teacher, &lse_student,
                       &diag_delta, &row_kl, nullptr, &rope, true, loss,
                       static_cast<char*>(reserve), &off, static_cast<double*>(workspace),
                       stream);
}

lard_status lard_relkl_rope_bwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                const void* reserve, size_t reserve_bytes,
                                const float* lse_teacher, const float* lse_student,
                                const float* diag_delta, const float* grad_loss,
                                const lard_grad_desc* grad, void* dx_student, void* workspace,
                                size_t workspace_bytes, void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if ((s = check_rope(rope)) != LARD_OK) return s;
  if (!reserve || !aligned(reserve, 256)) return LARD_ERR_INVALID_ARGUMENT;
  if ((s = check_bwd_state(lse_teacher, lse_student, diag_delta, true)) != LARD_OK) return s;
  if (!grad_loss || !aligned(grad_loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
  if ((s = check_grad(desc, grad, dx_student)) != LARD_OK) return s;
  if (reserve_bytes < reserve_total(desc, Path::kRope)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  s = check_bwd_workspace(workspace, workspace_bytes, bwd_workspace(1, &desc));
  if (s != LARD_OK) return s;
  const size_t off = 0;
  const void* none = nullptr;
  return run_group_bwd(1, &desc, &none, &none, &lse_teacher, &lse_student, &diag_delta, &rope,
                       true, static_cast<const char*>(reserve), &off, grad_loss, &grad,
                       &dx_student, static_cast<float*>(workspace), stream);
}

size_t lard_relkl_cross_reserve_size(const lard_relkl_desc* desc, lard_status* status) {
  const lard_status s = check_desc(desc);
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return reserve_total(desc, Path::kCross);
}

lard_status lard_relkl_cross_fwd(const lard_relkl_desc* desc, const lard_cross_desc* keys,
                                 const lard_rope_desc* rope, const void* a_teacher,
                                 const void* b_teacher, const void* a_student,
                                 const void* b_student, float* lse_teacher, float* lse_student,
                                 float* row_kl, float* loss, void* reserve, size_t reserve_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if ((s = check_cross(desc, keys)) != LARD_OK) return s;
  if (rope && (s = check_rope(rope)) != LARD_OK) return s;
  if ((s = check_inputs(a_teacher, a_student)) != LARD_OK) return s;
  if ((s = check_inputs(b_teacher, b_student)) != LARD_OK) return s;
  if ((s = check_fwd_outputs(lse_teacher, lse_student, nullptr, row_kl)) != LARD_OK) return s;
  if (!loss || !workspace || !reserve) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 8) || !aligned(reserve, 256) || !aligned(loss, 4))
    return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fwd_workspace(1, &desc)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const ReserveLayout R = reserve_of(desc, Path::kCross);
  if (reserve_bytes < R.total) return LARD_ERR_WORKSPACE_TOO_SMALL;
  const bool bf16 = desc->dtype == LARD_BF16;
  char* rb = static_cast<char*>(reserve);
  MapTable maps;
  build_maps(maps, 1, &desc);

  // 1. copies (rotated when tables are given) of A and B of both sides: one launch with
  //    A and B as two members of the same problem
  PrepLaunch P;
  launch_init(P);
  prep_member(P, desc, a_teacher, desc->t_stride_b, desc->t_stride_h, desc->t_stride_n,
              a_student, desc->s_stride_b, desc->s_stride_h, desc->s_stride_n, rope,
              rb + R.x_t, rb + R.x_s);
  prep_member(P, desc, b_teacher, keys->bt_stride_b, keys->bt_stride_h, keys->bt_stride_n,
              b_student, keys->bs_stride_b, keys->bs_stride_h, keys->bs_stride_n, rope,
              rb + R.y_t, rb + R.y_s);
  memcpy(P.head_map, maps.v, sizeof(maps.v));
  P.m[0].map_off = P.m[1].map_off = maps.off[0];
  if (launch_rope_prep(P, bf16, desc->d, stream, /*f16_images=*/true) != 0) return LARD_ERR_HIP;

  // 2. the forward: own rows from the A copies, key tiles from the B copies
  FwdLaunch F;
  launch_init(F);
  FwdArgs& a = add_member(F, (int)fwd_partials(desc));
  fwd_copies(a, desc, rb + R.x_t, rb + R.x_s, rb + R.y_t, rb + R.y_s);
  fwd_common(a, desc, lse_teacher, lse_student, nullptr, row_kl,
             static_cast<double*>(workspace));
  identity_maps(F);
  const LossOut lo = loss_out(F, static_cast<double*>(workspace), loss, nullptr);
  const int e = launch_fwd(F, bf16, desc->d, desc->causal == 1, lo, stream, /*cross=*/true);
  return e == 0 ? LARD_OK : LARD_ERR_HIP;
}

lard_status lard_relkl_cross_bwd(const lard_relkl_desc* desc, const lard_rope_desc* rope,
                                 const void* reserve, size_t reserve_bytes,
                                 const float* lse_teacher, const float* lse_student,
                                 const float* grad_loss, const lard_grad_desc* grad_a,
                                 void* da_student, const lard_grad_desc* grad_b,
                                 void* db_student, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  lard_status s = check_desc(desc);
  if (s != LARD_OK) return s;
  if (rope && (s = check_rope(rope)) != LARD_OK) return s;
  if (!reserve || !aligned(reserve, 256)) return LARD_ERR_INVALID_ARGUMENT;
  if ((s = check_bwd_state(lse_teacher, lse_student, nullptr, false)) != LARD_OK) return s;
  if (!grad_loss || !aligned(grad_loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
  if ((s = check_grad(desc, grad_a, da_student)) != LARD_OK) return s;
  if ((s = check_grad(desc, grad_b, db_student)) != LARD_OK) return s;
  const ReserveLayout R = reserve_of(desc, Path::kCross);
  if (reserve_bytes < R.total) return LARD_ERR_WORKSPACE_TOO_SMALL;
  s = check_bwd_workspace(workspace, workspace_bytes, bwd_workspace(1, &desc));
  if (s != LARD_OK) return s;
  const char* rb = static_cast<const char*>(reserve);
  const int splits = choose_splits(1, &desc);
  MapTable maps;
  build_maps(maps, 1, &desc);
  float* part = static_cast<float*>(workspace);

  // Both passes use the statistics of the query rows (rows of A).
  auto pass = [&](size_t own_t, size_t own_s, size_t stg_t, size_t stg_s,
                  const lard_grad_desc* g, void* dx, int mode) {
    BwdLaunch L;
    launch_init(L);
    BwdArgs& a = add_member(L, bwd_workgroups(desc, splits));
    bwd_copies(a, rb, own_t, own_s, stg_t, stg_s);
    bwd_common(a, desc, lse_teacher, lse_student, splits, nullptr, grad_loss, g, dx, part);
    if (rope) {
      a.rope_cos = rope->cos_student;
      a.rope_sin = rope->sin_student;
    }
    use_maps(L, maps);  // output placement only: operands are read per unit
    return run_bwd(L, &desc, g->dtype == LARD_FP32, mode, stream);
  };
  // dA: own rows of A, staged rows of B, row terms
  s = pass(R.x_t, R.x_s, R.y_t, R.y_s, grad_a, da_student, 1);
  if (s != LARD_OK) return s;
  // dB: own rows of B, staged rows of A with their statistics, column terms
  return pass(R.y_t, R.y_s, R.x_t, R.x_s, grad_b, db_student, 2);
}

// ------------------------------------------------------------------ grouped entry points
size_t lard_relkl_group_reserve_size(int n, const lard_relkl_member* members, int with_rope,
                                     lard_status* status) {
  const lard_relkl_desc* d[LARD_MAX_GROUP];
  lard_status s = check_group(n, members, d);
  if (s == LARD_OK && with_rope != 0 && with_rope != 1) s = LARD_ERR_INVALID_ARGUMENT;
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return group_reserve(n, d, with_rope ? Path::kRope : Path::kPlain, nullptr);
}

size_t lard_relkl_group_workspace_size(int n, const lard_relkl_member* members, int pass,
                                       lard_status* status) {
  const lard_relkl_desc* d[LARD_MAX_GROUP];
  lard_status s = check_group(n, members, d);
  if (s == LARD_OK && pass != 0 && pass != 1) s = LARD_ERR_INVALID_ARGUMENT;
  if (status) *status = s;
  if (s != LARD_OK) return 0;
  return pass == 0 ? fwd_workspace(n, d) : bwd_workspace(n, d);
}

lard_status lard_relkl_group_fwd(int n, const lard_relkl_member* members, int with_rope,
                                 float* loss, void* reserve, size_t reserve_bytes,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const lard_relkl_desc* d[LARD_MAX_GROUP];
  lard_status s = check_group(n, members, d);
  if (s != LARD_OK) return s;
  if (with_rope != 0 && with_rope != 1) return LARD_ERR_INVALID_ARGUMENT;
  const void* xt[LARD_MAX_GROUP];
  const void* xs[LARD_MAX_GROUP];
  float* lt[LARD_MAX_GROUP];
  float* ls[LARD_MAX_GROUP];
  float* dg[LARD_MAX_GROUP];
  float* kl[LARD_MAX_GROUP];
  float* ml[LARD_MAX_GROUP];
  const lard_rope_desc* rp[LARD_MAX_GROUP];
  for (int k = 0; k < n; ++k) {
    const lard_relkl_member& m = members[k];
    if ((s = check_inputs(m.x_teacher, m.x_student)) != LARD_OK) return s;
    if ((s = check_fwd_outputs(m.lse_teacher, m.lse_student, m.diag_delta, m.row_kl)) != LARD_OK)
      return s;
    if (m.loss && !aligned(m.loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
    if (with_rope && (s = check_rope(&m.rope)) != LARD_OK) return s;
    xt[k] = m.x_teacher;
    xs[k] = m.x_student;
    lt[k] = m.lse_teacher;
    ls[k] = m.lse_student;
    dg[k] = m.diag_delta;
    kl[k] = m.row_kl;
    ml[k] = m.loss;
    rp[k] = &m.rope;
  }
  if (!loss || !workspace) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 8) || !aligned(loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < fwd_workspace(n, d)) return LARD_ERR_WORKSPACE_TOO_SMALL;
  size_t off[LARD_MAX_GROUP];
  const Path path = with_rope ? Path::kRope : Path::kPlain;
  const size_t need = group_reserve(n, d, path, off);
  if (need > 0 && (!reserve || !aligned(reserve, 256))) return LARD_ERR_INVALID_ARGUMENT;
  if (reserve_bytes < need) return LARD_ERR_WORKSPACE_TOO_SMALL;
  return run_group_fwd(n, d, xt, xs, lt, ls, dg, kl, ml, rp, with_rope == 1, loss,
                       static_cast<char*>(reserve), off, static_cast<double*>(workspace),
                       stream);
}

lard_status lard_relkl_group_bwd(int n, const lard_relkl_member* members, int with_rope,
                                 const void* reserve, size_t reserve_bytes,
                                 const float* grad_loss, const lard_grad_desc* grads,
                                 void* const* dx_student, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const lard_relkl_desc* d[LARD_MAX_GROUP];
  lard_status s = check_group(n, members, d);
  if (s != LARD_OK) return s;
  if (with_rope != 0 && with_rope != 1) return LARD_ERR_INVALID_ARGUMENT;
  if (!grad_loss || !grads || !dx_student) return LARD_ERR_INVALID_ARGUMENT;
  if (!aligned(grad_loss, 4)) return LARD_ERR_INVALID_ARGUMENT;
  const void* xt[LARD_MAX_GROUP];
  const void* xs[LARD_MAX_GROUP];
  const float* lt[LARD_MAX_GROUP];
  const float* ls[LARD_MAX_GROUP];
  const float* dg[LARD_MAX_GROUP];
  const lard_rope_desc* rp[LARD_MAX_GROUP];
  const lard_grad_desc* g[LARD_MAX_GROUP];
  void* dx[LARD_MAX_GROUP];
  for (int k = 0; k < n; ++k) {
    const lard_relkl_member& m = members[k];
    if (!with_rope && (s = check_inputs(m.x_teacher, m.x_student)) != LARD_OK) return s;
    if (with_rope && (s = check_rope(&m.rope)) != LARD_OK) return s;
    if ((s = check_bwd_state(m.lse_teacher, m.lse_student, m.diag_delta, true)) != LARD_OK)
      return s;
    if ((s = check_grad(d[k], &grads[k], dx_student[k])) != LARD_OK) return s;
    if (grads[k].dtype != grads[0].dtype) return LARD_ERR_INVALID_ARGUMENT;
    xt[k] = m.x_teacher;
    xs[k] = m.x_student;
    lt[k] = m.lse_teacher;
    ls[k] = m.lse_student;
    dg[k] = m.diag_delta;
    rp[k] = &m.rope;
    g[k] = &grads[k];
    dx[k] = dx_student[k];
  }
  size_t off[LARD_MAX_GROUP];
  const Path path = with_rope ? Path::kRope : Path::kPlain;
  const size_t need = group_reserve(n, d, path, off);
  if (need > 0 && (!reserve || !aligned(reserve, 256))) return LARD_ERR_INVALID_ARGUMENT;
  if (reserve_bytes < need) return LARD_ERR_WORKSPACE_TOO_SMALL;
  s = check_bwd_workspace(workspace, workspace_bytes, bwd_workspace(n, d));
  if (s != LARD_OK) return s;
  return run_group_bwd(n, d, xt, xs, lt, ls, dg, rp, with_rope == 1,
                       static_cast<const char*>(reserve), off, grad_loss, g, dx,
                       static_cast<float*>(workspace), stream);
}

}  // extern "C"
