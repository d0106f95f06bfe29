// C ABI of the Mamba-3 forward path: validation and dispatch.
//
// Validation mirrors the rules of the oarust 0.8.6 page
// src/rs/ml/matrix/mamba3.rs: Geometry::resolve (SISO), MimoGeometry::resolve
// (MIMO, without its P*N <= 4096 capacity cap), PreprocessGeometry::resolve
// and the sequence_length == 1 rule of dispatch_mamba3_siso_step, plus the
// u32 element-count limits those functions apply.  Every rule is checked on
// the host before any HIP call, so a rejected call touches no device memory
// and does not initialise the HIP runtime.
#include "../../include/m3.h"
#include "launch.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

constexpr uint64_t kU32 = 0xffffffffull;

// Product of extents, false on overflow of uint32 (the stable shader ABI width).
bool count_u32(std::initializer_list<uint64_t> ext) {
  uint64_t c = 1;
  for (uint64_t e : ext) {
    if (e != 0 && c > kU32 / e) return false;
    c *= e;
  }
  return c <= kU32;
}

struct Resolved {
  m3::ScanGeom g;
};

// Shared rule set of the scan geometry, one rule at a time, so that the
// message names the rule that failed.  `mimo` selects the multi-input rules
// (rank 1..8 and an optional output norm) instead of the single-input ones
// (rank exactly 1, no output norm).
int resolve_scan(const char* op, const m3_ssm_config& cfg, bool mimo, m3::ScanGeom* out) {
  const uint32_t G = cfg.num_groups == 0 ? cfg.num_heads : cfg.num_groups;
  const struct {
    const char* name;
    uint32_t v;
  } flags[] = {{"has_z", cfg.has_z}, {"has_d", cfg.has_d}, {"has_output_norm", cfg.has_output_norm}};
  for (const auto& f : flags)
    if (f.v > 1) return fail(M3_ERR_INVALID_ARGUMENT, "%s: flag %s is %u; a flag is 0 or 1", op, f.name, f.v);
  const struct {
    const char* name;
    uint32_t v;
  } extents[] = {{"batch_size", cfg.batch_size}, {"sequence_length", cfg.sequence_length},
                 {"num_heads", cfg.num_heads}, {"head_dim", cfg.head_dim}, {"state_size", cfg.state_size}};
  for (const auto& e : extents)
    if (e.v == 0) return fail(M3_ERR_INVALID_ARGUMENT, "%s: %s is 0; every extent must be at least 1", op, e.name);
  if (cfg.num_heads % G != 0)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: num_groups %u does not divide num_heads %u", op, G, cfg.num_heads);
  if (cfg.head_dim > 128)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: head_dim %u is above the limit of 128", op, cfg.head_dim);
  if (cfg.state_size > 128)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: state_size %u is above the limit of 128", op, cfg.state_size);
  if (cfg.num_rope_angles > 64)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: num_rope_angles %u is above the limit of 64", op,
                cfg.num_rope_angles);
  if (2ull * cfg.num_rope_angles > cfg.state_size)
    return fail(M3_ERR_INVALID_ARGUMENT,
                "%s: the %u rotary pairs need 2 * num_rope_angles = %u state coordinates, but state_size is %u",
                op, cfg.num_rope_angles, 2 * cfg.num_rope_angles, cfg.state_size);
  if (mimo) {
    if (cfg.mimo_rank < 1 || cfg.mimo_rank > 8)
      return fail(M3_ERR_INVALID_ARGUMENT, "%s: mimo_rank %u is outside 1..8", op, cfg.mimo_rank);
  } else {
    if (cfg.mimo_rank != 1)
      return fail(M3_ERR_INVALID_ARGUMENT, "%s: mimo_rank is %u; the single-input scan takes rank 1 only", op,
                  cfg.mimo_rank);
    if (cfg.has_output_norm != 0)
      return fail(M3_ERR_INVALID_ARGUMENT,
                  "%s: has_output_norm is set; the output norm belongs to the multi-input scan only", op);
  }
  const uint64_t B = cfg.batch_size, L = cfg.sequence_length, H = cfg.num_heads, P = cfg.head_dim,
                 N = cfg.state_size, A = cfg.num_rope_angles, R = mimo ? cfg.mimo_rank : 1;
  const struct {
    const char* name;
    bool ok;
  } counts[] = {{"c / b", count_u32({B, L, R * G, N})}, {"x / z / out", count_u32({B, L, H, P})},
                {"adt / dt / trap", count_u32({B, L, H})}, {"angle", count_u32({B, L, A})},
                {"c_bias / b_bias", count_u32({H, R, N})}, {"mimo weight", count_u32({H, R, P})},
                {"batch * heads", count_u32({B, H})}};
  for (const auto& c : counts)
    if (!c.ok)
      return fail(M3_ERR_INVALID_ARGUMENT, "%s: the %s element count does not fit in u32", op, c.name);
  out->B = cfg.batch_size;
  out->L = cfg.sequence_length;
  out->H = cfg.num_heads;
  out->G = G;
  out->P = cfg.head_dim;
  out->N = cfg.state_size;
  out->A = cfg.num_rope_angles;
  out->R = (uint32_t)R;
  out->has_z = cfg.has_z;
  out->has_d = cfg.has_d;
  out->has_norm = mimo ? cfg.has_output_norm : 0;
  return M3_OK;
}

int check_ptrs(const char* op, std::initializer_list<std::pair<const char*, const void*>> ptrs) {
  for (const auto& pr : ptrs)
    if (pr.second == nullptr) return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand %s is NULL", op, pr.first);
  return M3_OK;
}

int hip_status(const char* op, hipError_t e) {
  if (e == hipSuccess) return M3_OK;
  return fail(M3_ERR_HIP, "%s: HIP error %d (%s)", op, (int)e, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* m3_last_error(void) { return g_err; }

void m3_set_profile_events(void* start_event, void* stop_event) {
  m3::ProfileEvents& pe = m3::profile_events();
  const bool on = start_event != nullptr && stop_event != nullptr;
  pe.start = on ? static_cast<hipEvent_t>(start_event) : nullptr;
  pe.stop = on ? static_cast<hipEvent_t>(stop_event) : nullptr;
}

const char* m3_version(void) { return "m3 0.2.0 gfx950"; }

void m3_set_scan_segments(uint32_t segments) { m3::set_forced_segments(segments); }

}  // extern "C"

namespace {

// Preprocess geometry rules shared by the forward and the backward, checked
// one at a time so that the message names the rule that failed.
int resolve_pre(const char* op, uint32_t rows, const m3_preprocess_config& cfg, m3::PreGeom* out) {
  const struct {
    const char* name;
    uint32_t v;
  } extents[] = {{"rows", rows}, {"inner_size", cfg.inner_size}, {"state_size", cfg.state_size},
                 {"num_heads", cfg.num_heads}, {"num_groups", cfg.num_groups}, {"mimo_rank", cfg.mimo_rank}};
  for (const auto& e : extents)
    if (e.v == 0) return fail(M3_ERR_INVALID_ARGUMENT, "%s: %s is 0; every extent must be at least 1", op, e.name);
  if (2ull * cfg.num_rope_angles > cfg.state_size)
    return fail(M3_ERR_INVALID_ARGUMENT,
                "%s: the %u rotary pairs need 2 * num_rope_angles = %u state coordinates, but state_size is %u",
                op, cfg.num_rope_angles, 2 * cfg.num_rope_angles, cfg.state_size);
  const struct {
    const char* name;
    float v;
  } bounds[] = {{"epsilon", cfg.epsilon}, {"dt_min", cfg.dt_min}, {"dt_max", cfg.dt_max}, {"a_floor", cfg.a_floor}};
  for (const auto& b : bounds)
    if (!std::isfinite(b.v)) return fail(M3_ERR_INVALID_ARGUMENT, "%s: %s is not a finite number", op, b.name);
  // dt_max needs no sign rule of its own: it is at least dt_min
  for (const auto& b : {bounds[0], bounds[1], bounds[3]})
    if (b.v <= 0.f)
      return fail(M3_ERR_INVALID_ARGUMENT, "%s: %s is %g; it must be above zero", op, b.name, (double)b.v);
  if (cfg.dt_min > cfg.dt_max)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: dt_min %g is above dt_max %g", op, (double)cfg.dt_min,
                (double)cfg.dt_max);
  const uint64_t I = cfg.inner_size, N = cfg.state_size, H = cfg.num_heads,
                 A = cfg.num_rope_angles, GR = (uint64_t)cfg.num_groups * cfg.mimo_rank;
  const uint64_t M = GR * N;
  const uint64_t W = 2 * I + 2 * M + 3 * H + A;
  if (GR > kU32 || M > kU32 || W > kU32 || !count_u32({rows, W}) || !count_u32({rows, I}) ||
      !count_u32({rows, M}) || !count_u32({rows, H}) || !count_u32({rows, A}))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: projected width or an element count exceeds u32", op);
  *out = m3::PreGeom{rows, cfg.inner_size, cfg.state_size, cfg.num_heads, cfg.num_rope_angles,
                     cfg.num_groups, cfg.mimo_rank, cfg.epsilon, cfg.dt_min, cfg.dt_max, cfg.a_floor};
  return M3_OK;
}

}  // namespace

extern "C" {

int m3_preprocess(const float* projected, const float* dt_bias, uint32_t rows,
                  m3_preprocess_config cfg, float* x, float* z, float* bh, float* ch, float* dt,
                  float* adt, float* trap, float* angle, void* stream) {
  const char* op = "m3_preprocess";
  clear_error();
  m3::PreGeom g{};
  int st = resolve_pre(op, rows, cfg, &g);
  if (st) return st;
  st = check_ptrs(op, {{"projected", projected}, {"dt_bias", dt_bias}, {"x", x}, {"z", z},
                       {"bh", bh}, {"ch", ch}, {"dt", dt}, {"adt", adt}, {"trap", trap}});
  if (st) return st;
  if (g.A > 0 && angle == nullptr) return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand angle is NULL", op);
  m3::PreOperands o{projected, dt_bias, x, z, bh, ch, dt, adt, trap, angle};
  return hip_status(op, m3::launch_preprocess(g, o, static_cast<hipStream_t>(stream)));
}

int m3_preprocess_bwd(const float* projected, const float* dt_bias, uint32_t rows,
                      m3_preprocess_config cfg, const float* g_x, const float* g_z, const float* g_bh,
                      const float* g_ch, const float* g_dt, const float* g_adt, const float* g_trap,
                      const float* g_angle, float* d_projected, float* d_dt_bias, void* stream) {
  const char* op = "m3_preprocess_bwd";
  clear_error();
  m3::PreGeom g{};
  int st = resolve_pre(op, rows, cfg, &g);
  if (st) return st;
  st = check_ptrs(op, {{"projected", projected}, {"dt_bias", dt_bias}, {"d_projected", d_projected},
                       {"d_dt_bias", d_dt_bias}});
  if (st) return st;
  m3::PreBwdOperands o{projected, dt_bias, g_x, g_z, g_bh, g_ch, g_dt, g_adt, g_trap,
                       g.A > 0 ? g_angle : nullptr, d_projected, d_dt_bias};
  return hip_status(op, m3::launch_preprocess_bwd(g, o, static_cast<hipStream_t>(stream)));
}

size_t m3_siso_bwd_workspace_bytes(m3_ssm_config cfg) {
  m3::ScanGeom g{};
  if (resolve_scan("m3_siso_bwd_workspace_bytes", cfg, false, &g) != M3_OK) return 0;
  return m3::siso_bwd_workspace_floats(g) * sizeof(float);
}

int m3_siso_bwd(const float* dout, const float* c, const float* b, const float* x, const float* z,
                const float* adt, const float* dt, const float* trap, const float* angle,
                const float* c_bias, const float* b_bias, const float* d, m3_ssm_config cfg,
                float* d_c, float* d_b, float* d_x, float* d_z, float* d_adt, float* d_dt,
                float* d_trap, float* d_angle, float* d_c_bias, float* d_b_bias, float* d_d,
                void* workspace, size_t workspace_bytes, void* stream) {
  const char* op = "m3_siso_bwd";
  clear_error();
  m3::ScanGeom g{};
  int st = resolve_scan(op, cfg, false, &g);
  if (st) return st;
  st = check_ptrs(op, {{"dout", dout}, {"c", c}, {"b", b}, {"x", x}, {"z", z}, {"adt", adt},
                       {"dt", dt}, {"trap", trap}, {"c_bias", c_bias}, {"b_bias", b_bias}, {"d", d},
                       {"d_c", d_c}, {"d_b", d_b}, {"d_x", d_x}, {"d_z", d_z}, {"d_adt", d_adt},
                       {"d_dt", d_dt}, {"d_trap", d_trap}, {"d_c_bias", d_c_bias},
                       {"d_b_bias", d_b_bias}, {"d_d", d_d}});
  if (st) return st;
  if (g.A > 0 && (angle == nullptr || d_angle == nullptr))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand angle or d_angle is NULL", op);
  if (!m3::siso_bwd_fits(g))
    return fail(M3_ERR_UNSUPPORTED, "%s: %u heads per group with state_size %u exceed the LDS of the "
                "backward group reduction", op, g.H / g.G, g.N);
  const size_t need = m3::siso_bwd_workspace_floats(g) * sizeof(float);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: workspace of %zu bytes required, %zu given", op, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  m3::ScanOperands o{c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     nullptr, nullptr, nullptr, nullptr, nullptr};
  m3::BwdOperands go{dout, d_c, d_b, d_x, d_z, d_adt, d_dt, d_trap, d_angle, d_c_bias, d_b_bias, d_d};
  return hip_status(op, m3::launch_siso_bwd(g, o, go, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Fused preprocess -> scan: the two configs must describe one geometry.
struct PackedPlan {
  m3::ScanGeom g;
  m3::PreGeom pg;
  m3::ScanPlan plan;
  size_t o_bh, o_ch, o_dt, o_adt, o_scan, total_bytes;
  uint32_t W, I, M;
};

int resolve_packed(const char* op, const m3_preprocess_config& pcfg, const m3_ssm_config& cfg, PackedPlan* pp) {
  int st = resolve_scan(op, cfg, false, &pp->g);
  if (st) return st;
  const m3::ScanGeom& g = pp->g;
  if (!count_u32({g.B, g.L})) return fail(M3_ERR_INVALID_ARGUMENT, "%s: batch_size * sequence_length exceeds u32", op);
  st = resolve_pre(op, g.B * g.L, pcfg, &pp->pg);
  if (st) return st;
  if ((uint64_t)pcfg.inner_size != (uint64_t)g.H * g.P)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: inner_size %u differs from num_heads * head_dim = %u", op,
                pcfg.inner_size, g.H * g.P);
  const struct {
    const char* name;
    uint32_t pre, scan;
  } same[] = {{"state_size", pcfg.state_size, g.N}, {"num_heads", pcfg.num_heads, g.H},
              {"num_rope_angles", pcfg.num_rope_angles, g.A}, {"num_groups", pcfg.num_groups, g.G}};
  for (const auto& m : same)
    if (m.pre != m.scan)
      return fail(M3_ERR_INVALID_ARGUMENT, "%s: %s is %u in the preprocess config but %u in the scan config", op,
                  m.name, m.pre, m.scan);
  if (pcfg.mimo_rank != 1)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: the preprocess config has mimo_rank %u; the fused call is rank 1",
                op, pcfg.mimo_rank);
  pp->I = pcfg.inner_size;
  pp->M = g.G * g.N;
  pp->W = 2 * pp->I + 2 * pp->M + 3 * g.H + g.A;
  pp->plan = m3::plan_siso(g);
  const size_t rows = (size_t)g.B * g.L;
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t o = off;
    off += (floats + 63) / 64 * 64;  // 256-byte aligned pieces
    return o;
  };
  pp->o_bh = take(rows * pp->M);
  pp->o_ch = take(rows * pp->M);
  pp->o_dt = take(rows * g.H);
  pp->o_adt = take(rows * g.H);
  pp->o_scan = off;
  pp->total_bytes = off * sizeof(float) + m3::plan_workspace_bytes(pp->plan);
  return M3_OK;
}

}  // namespace

extern "C" {

size_t m3_siso_fwd_packed_workspace_bytes(m3_preprocess_config pcfg, m3_ssm_config cfg) {
  PackedPlan pp{};
  if (resolve_packed("m3_siso_fwd_packed_workspace_bytes", pcfg, cfg, &pp) != M3_OK) return 0;
  return pp.total_bytes;
}

int m3_siso_fwd_packed(const float* projected, const float* dt_bias, const float* c_bias,
                       const float* b_bias, const float* d, m3_preprocess_config pcfg,
                       m3_ssm_config cfg, float* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  const char* op = "m3_siso_fwd_packed";
  clear_error();
  PackedPlan pp{};
  int st = resolve_packed(op, pcfg, cfg, &pp);
  if (st) return st;
  st = check_ptrs(op, {{"projected", projected}, {"dt_bias", dt_bias}, {"c_bias", c_bias},
                       {"b_bias", b_bias}, {"d", d}, {"out", out}, {"workspace", workspace}});
  if (st) return st;
  if (workspace_bytes < pp.total_bytes)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: workspace of %zu bytes required, %zu given", op,
                pp.total_bytes, workspace_bytes);
  float* ws = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  m3::PreOperands po{projected, dt_bias, nullptr, nullptr, ws + pp.o_bh, ws + pp.o_ch,
                     ws + pp.o_dt, ws + pp.o_adt, nullptr, nullptr};
  st = hip_status(op, m3::launch_preprocess_derived(pp.pg, po, s));
  if (st) return st;
  const m3::ScanGeom& g = pp.g;
  const uint32_t o_tr = 2 * pp.I + 2 * pp.M + 2 * g.H;
  m3::ScanOperands o{ws + pp.o_ch, ws + pp.o_bh, projected + pp.I, projected, ws + pp.o_adt, ws + pp.o_dt,
                     projected + o_tr, g.A > 0 ? projected + o_tr + g.H : nullptr, c_bias, b_bias, d,
                     nullptr, nullptr, nullptr, nullptr, out, pp.W, pp.W, pp.W};
  void* scan_ws = m3::plan_workspace_bytes(pp.plan) > 0 ? static_cast<void*>(ws + pp.o_scan) : nullptr;
  return hip_status(op, m3::launch_siso_fwd(g, o, pp.plan, scan_ws, s));
}

size_t m3_mimo_bwd_workspace_bytes(m3_ssm_config cfg) {
  m3::ScanGeom g{};
  if (resolve_scan("m3_mimo_bwd_workspace_bytes", cfg, true, &g) != M3_OK) return 0;
  return m3::mimo_bwd_workspace_floats(g) * sizeof(float);
}

int m3_mimo_bwd(const float* dout, const float* c, const float* b, const float* x, const float* z,
                const float* adt, const float* dt, const float* trap, const float* angle,
                const float* c_bias, const float* b_bias, const float* d, const float* mimo_x,
                const float* mimo_z, const float* mimo_o, const float* norm_weight, m3_ssm_config cfg,
                float* d_c, float* d_b, float* d_x, float* d_z, float* d_adt, float* d_dt,
                float* d_trap, float* d_angle, float* d_c_bias, float* d_b_bias, float* d_d,
                float* d_mimo_x, float* d_mimo_z, float* d_mimo_o, float* d_norm_weight,
                void* workspace, size_t workspace_bytes, void* stream) {
  const char* op = "m3_mimo_bwd";
  clear_error();
  m3::ScanGeom g{};
  int st = resolve_scan(op, cfg, true, &g);
  if (st) return st;
  st = check_ptrs(op, {{"dout", dout}, {"c", c}, {"b", b}, {"x", x}, {"z", z}, {"adt", adt},
                       {"dt", dt}, {"trap", trap}, {"c_bias", c_bias}, {"b_bias", b_bias}, {"d", d},
                       {"mimo_x", mimo_x}, {"mimo_z", mimo_z}, {"mimo_o", mimo_o},
                       {"norm_weight", norm_weight}, {"d_c", d_c}, {"d_b", d_b}, {"d_x", d_x},
                       {"d_z", d_z}, {"d_adt", d_adt}, {"d_dt", d_dt}, {"d_trap", d_trap},
                       {"d_c_bias", d_c_bias}, {"d_b_bias", d_b_bias}, {"d_d", d_d},
                       {"d_mimo_x", d_mimo_x}, {"d_mimo_z", d_mimo_z}, {"d_mimo_o", d_mimo_o},
                       {"d_norm_weight", d_norm_weight}});
  if (st) return st;
  if (g.A > 0 && (angle == nullptr || d_angle == nullptr))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand angle or d_angle is NULL", op);
  if (!m3::mimo_bwd_fits(g))
    return fail(M3_ERR_UNSUPPORTED, "%s: %u heads per group at rank %u with state_size %u exceed the LDS of the "
                "backward kernels", op, g.H / g.G, g.R, g.N);
  const size_t need = m3::mimo_bwd_workspace_floats(g) * sizeof(float);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: workspace of %zu bytes required, %zu given", op, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  m3::ScanOperands o{c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     mimo_x, mimo_z, mimo_o, norm_weight, nullptr};
  m3::BwdOperands go{dout, d_c, d_b, d_x, d_z, d_adt, d_dt, d_trap, d_angle, d_c_bias, d_b_bias, d_d,
                     d_mimo_x, d_mimo_z, d_mimo_o, d_norm_weight};
  return hip_status(op, m3::launch_mimo_bwd(g, o, go, workspace, static_cast<hipStream_t>(stream)));
}

size_t m3_siso_fwd_workspace_bytes(m3_ssm_config cfg) {
  m3::ScanGeom g{};
  if (resolve_scan("m3_siso_fwd_workspace_bytes", cfg, false, &g) != M3_OK) return 0;
  return m3::plan_workspace_bytes(m3::plan_siso(g));
}

size_t m3_mimo_fwd_workspace_bytes(m3_ssm_config cfg) {
  m3::ScanGeom g{};
  if (resolve_scan("m3_mimo_fwd_workspace_bytes", cfg, true, &g) != M3_OK) return 0;
  return m3::plan_workspace_bytes(m3::plan_mimo(g));
}

int m3_siso_fwd(const float* c, const float* b, const float* x, const float* z, const float* adt,
                const float* dt, const float* trap, const float* angle, const float* c_bias,
                const float* b_bias, const float* d, m3_ssm_config cfg, float* out, void* workspace,
                size_t workspace_bytes, void* stream) {
  const char* op = "m3_siso_fwd";
  clear_error();
  m3::ScanGeom g{};
  int st = resolve_scan(op, cfg, false, &g);
  if (st) return st;
  st = check_ptrs(op, {{"c", c}, {"b", b}, {"x", x}, {"z", z}, {"adt", adt}, {"dt", dt},
                       {"trap", trap}, {"c_bias", c_bias}, {"b_bias", b_bias}, {"d", d}, {"out", out}});
  if (st) return st;
  if (g.A > 0 && angle == nullptr) return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand angle is NULL", op);
  const m3::ScanPlan plan = m3::plan_siso(g);
  const size_t need = m3::plan_workspace_bytes(plan);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: workspace of %zu bytes required, %zu given", op, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  m3::ScanOperands o{c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     nullptr, nullptr, nullptr, nullptr, out};
  return hip_status(op, m3::launch_siso_fwd(g, o, plan, workspace, static_cast<hipStream_t>(stream)));
}

int m3_mimo_fwd(const float* c, const float* b, const float* x, const float* z, const float* adt,
                const float* dt, const float* trap, const float* angle, const float* c_bias,
                const float* b_bias, const float* d, const float* mimo_x, const float* mimo_z,
                const float* mimo_o, const float* norm_weight, m3_ssm_config cfg, float* out,
                void* workspace, size_t workspace_bytes, void* stream) {
  const char* op = "m3_mimo_fwd";
  clear_error();
  m3::ScanGeom g{};
  int st = resolve_scan(op, cfg, true, &g);
  if (st) return st;
  st = check_ptrs(op, {{"c", c}, {"b", b}, {"x", x}, {"z", z}, {"adt", adt}, {"dt", dt},
                       {"trap", trap}, {"c_bias", c_bias}, {"b_bias", b_bias}, {"d", d},
                       {"mimo_x", mimo_x}, {"mimo_z", mimo_z}, {"mimo_o", mimo_o},
                       {"norm_weight", norm_weight}, {"out", out}});
  if (st) return st;
  if (g.A > 0 && angle == nullptr) return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand angle is NULL", op);
  const m3::ScanPlan plan = m3::plan_mimo(g);
  const size_t need = m3::plan_workspace_bytes(plan);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: workspace of %zu bytes required, %zu given", op, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  m3::ScanOperands o{c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     mimo_x, mimo_z, mimo_o, norm_weight, out};
  return hip_status(op, m3::launch_mimo_fwd(g, o, plan, workspace, static_cast<hipStream_t>(stream)));
}

int m3_siso_step(const float* c, const float* b, const float* x, const float* z, const float* adt,
                 const float* dt, const float* trap, const float* angle, const float* c_bias,
                 const float* b_bias, const float* d, float* ssm_state, float* angle_state,
                 float* k_state, float* v_state, m3_ssm_config cfg, float* out, void* stream) {
  const char* op = "m3_siso_step";
  clear_error();
  m3::ScanGeom g{};
  int st = resolve_scan(op, cfg, false, &g);
  if (st) return st;
  if (cfg.sequence_length != 1)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: sequence_length is %u; a decode step takes exactly one token", op,
                cfg.sequence_length);
  if (!count_u32({g.B, g.H, g.P, g.N}))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: state element count exceeds u32", op);
  st = check_ptrs(op, {{"c", c}, {"b", b}, {"x", x}, {"z", z}, {"adt", adt}, {"dt", dt},
                       {"trap", trap}, {"c_bias", c_bias}, {"b_bias", b_bias}, {"d", d},
                       {"ssm_state", ssm_state}, {"k_state", k_state}, {"v_state", v_state},
                       {"out", out}});
  if (st) return st;
  if (g.A > 0 && (angle == nullptr || angle_state == nullptr))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand angle or angle_state is NULL", op);
  m3::ScanOperands o{c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     nullptr, nullptr, nullptr, nullptr, out};
  m3::StepStates s{ssm_state, angle_state, k_state, v_state};
  return hip_status(op, m3::launch_siso_step(g, o, s, static_cast<hipStream_t>(stream)));
}

int m3_mimo_step(const float* c, const float* b, const float* x, const float* z, const float* adt,
                 const float* dt, const float* trap, const float* angle, const float* c_bias,
                 const float* b_bias, const float* d, const float* mimo_x, const float* mimo_z,
                 const float* mimo_o, const float* norm_weight, float* ssm_state, float* angle_state,
                 float* k_state, float* v_state, m3_ssm_config cfg, float* out, void* stream) {
  const char* op = "m3_mimo_step";
  clear_error();
  m3::ScanGeom g{};
  int st = resolve_scan(op, cfg, true, &g);
  if (st) return st;
  if (cfg.sequence_length != 1)
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: sequence_length is %u; a decode step takes exactly one token", op,
                cfg.sequence_length);
  if (!count_u32({g.B, g.H, g.P, g.N}) || !count_u32({g.B, g.H, g.R, g.N}) || !count_u32({g.B, g.H, g.R, g.P}))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: state element count exceeds u32", op);
  st = check_ptrs(op, {{"c", c}, {"b", b}, {"x", x}, {"z", z}, {"adt", adt}, {"dt", dt},
                       {"trap", trap}, {"c_bias", c_bias}, {"b_bias", b_bias}, {"d", d},
                       {"mimo_x", mimo_x}, {"mimo_z", mimo_z}, {"mimo_o", mimo_o},
                       {"norm_weight", norm_weight}, {"ssm_state", ssm_state}, {"k_state", k_state},
                       {"v_state", v_state}, {"out", out}});
  if (st) return st;
  if (g.A > 0 && (angle == nullptr || angle_state == nullptr))
    return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand angle or angle_state is NULL", op);
  m3::ScanOperands o{c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     mimo_x, mimo_z, mimo_o, norm_weight, out};
  m3::StepStates s{ssm_state, angle_state, k_state, v_state};
  return hip_status(op, m3::launch_mimo_step(g, o, s, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- m3_siso_fwd_noalloc: the scan's workspace in a fixed device array ------
//
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops): the segment summaries live in `scratch`, a file-scope
// device array that every GPU the library runs on holds until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): on the first call on a device, with
// that device current, hipGetSymbolAddress gives that device's own copy,
// and every later call on the device uses the kept pointer.
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

}  // namespace

extern "C" {

int m3_siso_fwd_noalloc(const float* c, const float* b, const float* x, const float* z, const float* adt,
                        const float* dt, const float* trap, const float* angle, const float* c_bias,
                        const float* b_bias, const float* d, m3_ssm_config cfg, float* out, void* stream) {
  const char* op = "m3_siso_fwd_noalloc";
  clear_error();
  m3::ScanGeom g{};
  int st = resolve_scan(op, cfg, false, &g);
  if (st) return st;
  st = check_ptrs(op, {{"c", c}, {"b", b}, {"x", x}, {"z", z}, {"adt", adt}, {"dt", dt},
                       {"trap", trap}, {"c_bias", c_bias}, {"b_bias", b_bias}, {"d", d}, {"out", out}});
  if (st) return st;
  if (g.A > 0 && angle == nullptr) return fail(M3_ERR_INVALID_ARGUMENT, "%s: operand angle is NULL", op);
  const m3::ScanPlan plan = m3::plan_siso(g);
  const size_t need = m3::plan_workspace_bytes(plan);
  if (need > kScratchBytes)
    return fail(M3_ERR_UNSUPPORTED, "%s: this geometry needs %zu bytes of scan workspace; the fixed scratch holds %zu",
                op, need, kScratchBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(op, e);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(M3_ERR_UNSUPPORTED, "%s: device %d is beyond the %d devices the scratch table covers", op, dev,
                kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev] {
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
    if (g_scratch_err[dev] != hipSuccess) (void)hipGetLastError();
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_status(op, g_scratch_err[dev]);
  m3::ScanOperands o{c, b, x, z, adt, dt, trap, angle, c_bias, b_bias, d,
                     nullptr, nullptr, nullptr, nullptr, out};
  void* ws = need > 0 ? g_scratch_ptr[dev] : nullptr;
  return hip_status(op, m3::launch_siso_fwd(g, o, plan, ws, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

