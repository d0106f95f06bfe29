// Internal launch interface between the C ABI (abi.cpp) and the HIP kernels.
// Geometry arriving here has already been validated by abi.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

struct ScanGeom {
  uint32_t B, L, H, G, P, N, A, R;
  uint32_t has_z, has_d, has_norm;
};

struct ScanOperands {
  const float *c, *b, *x, *z, *adt, *dt, *trap, *angle, *c_bias, *b_bias, *d;
  const float *mimo_x, *mimo_z, *mimo_o, *norm_weight;  // MIMO only
  float* out;
  // per-token strides of x / z, trap and angle in elements; 0 = dense layout
  // (H P, H, A).  Packed projection rows give all three the row width.
  uint32_t xs, ts, as;
};

struct StepStates {
  float *ssm, *angle, *k, *v;
};

struct PreGeom {
  uint32_t rows, I, N, H, A, G, R;
  float eps, dt_min, dt_max, a_floor;
};

struct PreOperands {
  const float *projected, *dt_bias;
  float *x, *z, *bh, *ch, *dt, *adt, *trap, *angle;
};

// Upstream gradient and the eleven gradient outputs of the SISO backward.
struct BwdOperands {
  const float* dout;
  float *d_c, *d_b, *d_x, *d_z, *d_adt, *d_dt, *d_trap, *d_angle, *d_c_bias, *d_b_bias, *d_d;
  float *d_mimo_x, *d_mimo_z, *d_mimo_o, *d_norm_weight;  // MIMO only
};

// Gradients of the eight preprocess outputs (any may be null: zero) and the
// two gradient outputs of the preprocess backward.
struct PreBwdOperands {
  const float *projected, *dt_bias;
  const float *g_x, *g_z, *g_bh, *g_ch, *g_dt, *g_adt, *g_trap, *g_angle;
  float *d_projected, *d_dt_bias;
};

// Chunked scan plan: chunk length, number of sequence segments.
struct ScanPlan {
  int chunk;
  int nseg;
  int seg_len;
  int npc;   // summary pieces per segment before the last
  int plen;  // tokens per summary piece (whole chunks)
  size_t ws_state_floats;
  size_t ws_aux_floats;
};

// Events recorded around the main scan kernel (measurement hook; may be null).
struct ProfileEvents {
  hipEvent_t start, stop;
};
ProfileEvents& profile_events();

// Compute units of the current HIP device, queried once per device (256, the
// MI355X count, when no device answers).  The scan plan sizes its sequence
// segments by it, so a workspace query and the call it sizes must run with
// the same device current.
int device_cu_count();
// Thread-local override of the scan plan's sequence-segment count: 0 is the
// automatic choice; n > 0 asks for n segments (fewer when the sequence has
// fewer whole chunks).
void set_forced_segments(uint32_t nseg);

ScanPlan plan_siso(const ScanGeom& g);
ScanPlan plan_mimo(const ScanGeom& g);
inline size_t plan_workspace_bytes(const ScanPlan& p) {
  return (p.ws_state_floats + p.ws_aux_floats) * sizeof(float);
}

hipError_t launch_siso_fwd(const ScanGeom& g, const ScanOperands& o, const ScanPlan& plan,
                           void* workspace, hipStream_t stream);
hipError_t launch_mimo_fwd(const ScanGeom& g, const ScanOperands& o, const ScanPlan& plan,
                           void* workspace, hipStream_t stream);
hipError_t launch_siso_step(const ScanGeom& g, const ScanOperands& o, const StepStates& s,
                            hipStream_t stream);
hipError_t launch_mimo_step(const ScanGeom& g, const ScanOperands& o, const StepStates& s,
                            hipStream_t stream);
hipError_t launch_preprocess(const PreGeom& g, const PreOperands& o, hipStream_t stream);
// Only the derived preprocess outputs (bh, ch, dt, adt); the other pointers of o are ignored.
hipError_t launch_preprocess_derived(const PreGeom& g, const PreOperands& o, hipStream_t stream);
hipError_t launch_preprocess_bwd(const PreGeom& g, const PreBwdOperands& o, hipStream_t stream);

size_t siso_bwd_workspace_floats(const ScanGeom& g);
bool siso_bwd_fits(const ScanGeom& g);  // LDS of the backward kernels fits one CU
hipError_t launch_siso_bwd(const ScanGeom& g, const ScanOperands& o, const BwdOperands& go, void* workspace,
                           hipStream_t stream);
size_t mimo_bwd_workspace_floats(const ScanGeom& g);
bool mimo_bwd_fits(const ScanGeom& g);
hipError_t launch_mimo_bwd(const ScanGeom& g, const ScanOperands& o, const BwdOperands& go, void* workspace,
                           hipStream_t stream);

}  // namespace m3
