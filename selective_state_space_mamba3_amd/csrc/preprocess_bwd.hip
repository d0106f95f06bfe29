// Backward of the fused Mamba-3 projection preprocess for gfx950:
// mamba3_preprocess_backward of the oarust 0.8.6 page
// src/rs/ml/matrix/mamba3.rs (gradients of projected and dt_bias from the
// gradients of the eight preprocess outputs; an output without a gradient
// counts as zero).
//
// Per packed row, in the column order z | x | B | C | dt | A | trap | angle:
//   z, x, trap, angle:  the output gradient passes through;
//   B, C rows (N wide): y = v r, r = (mean(v^2) + eps)^-1/2, so
//                       dv = r gy - v r^3 mean(gy v);
//   dt:  u = dt_raw + dt_bias, dt = clamp(softplus(u)), adt = -max(softplus(A_raw), a_floor) dt:
//        du = (g_dt - max(softplus(A_raw), a_floor) g_adt) sigmoid(u) where the clamp
//        passes softplus(u) through (inclusive bounds), else 0;
//   A:   dA_raw = -dt g_adt sigmoid(A_raw) where softplus(A_raw) >= a_floor, else 0.
// d dt_bias[h] = sum over rows of du, summed in a fixed order by a second kernel.
#include "common.h"
#include "launch.h"

namespace m3 {
namespace {

struct PreBwdK {
  const float *projected, *dt_bias;
  const float *g_x, *g_z, *g_bh, *g_ch, *g_dt, *g_adt, *g_trap, *g_angle;
  float *d_projected, *d_dt_bias;
  int rows, W, I, N, H, A, M;  // M = G*R*N
  float eps, dt_min, dt_max, a_floor;
};

__device__ __forceinline__ void pass_slice(const float* src, float* dst, int n, int tid, int nthr) {
  if (src)
    for (int i = tid; i < n; i += nthr) dst[i] = src[i];
  else
    for (int i = tid; i < n; i += nthr) dst[i] = 0.f;
}

__global__ __launch_bounds__(256) void preprocess_bwd_kernel(PreBwdK p) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const float* src = p.projected + (size_t)row * p.W;
  float* dst = p.d_projected + (size_t)row * p.W;
  const int I = p.I, M = p.M, N = p.N, H = p.H, A = p.A;
  pass_slice(p.g_z ? p.g_z + (size_t)row * I : nullptr, dst, I, tid, blockDim.x);
  pass_slice(p.g_x ? p.g_x + (size_t)row * I : nullptr, dst + I, I, tid, blockDim.x);
  const int o_dt = 2 * I + 2 * M;
  pass_slice(p.g_trap ? p.g_trap + (size_t)row * H : nullptr, dst + o_dt + 2 * H, H, tid, blockDim.x);
  pass_slice(p.g_angle ? p.g_angle + (size_t)row * A : nullptr, dst + o_dt + 3 * H, A, tid, blockDim.x);

  // RMS-norm adjoint, one wave per N-wide row of B then C
  const int nrow = M / N;
  for (int k = wave; k < 2 * nrow; k += nw) {
    const bool isc = k >= nrow;
    const int col = 2 * I + (isc ? M : 0) + (k - (isc ? nrow : 0)) * N;
    const float* gsrc = isc ? p.g_ch : p.g_bh;
    if (!gsrc) {
      for (int n = lane; n < N; n += 64) dst[col + n] = 0.f;
      continue;
    }
    const float* gy = gsrc + (size_t)row * M + (col - 2 * I - (isc ? M : 0));
    float sv = 0.f, sg = 0.f;
    for (int n = lane; n < N; n += 64) {
      const float v = src[col + n];
      sv = fmaf(v, v, sv);
      sg = fmaf(gy[n], v, sg);
    }
    sv = read_lane_f(scan64_f(sv), 63);
    sg = read_lane_f(scan64_f(sg), 63);
    const float r = 1.f / sqrtf(sv / (float)N + p.eps);
    const float c3 = r * r * r * (sg / (float)N);
    for (int n = lane; n < N; n += 64) dst[col + n] = fmaf(r, gy[n], -src[col + n] * c3);
  }

  // dt and A columns, one thread per head
  for (int h = tid; h < H; h += blockDim.x) {
    const float u = src[o_dt + h] + p.dt_bias[h];
    const float sp = softplusf_acc(u);
    const bool dt_pass = sp >= p.dt_min && sp <= p.dt_max;
    const float dtv = fminf(fmaxf(sp, p.dt_min), p.dt_max);
    const float ar = src[o_dt + H + h];
    const float spa = softplusf_acc(ar);
    const bool a_pass = spa >= p.a_floor;
    const float a_mag = fmaxf(spa, p.a_floor);
    const float gdt = p.g_dt ? p.g_dt[(size_t)row * H + h] : 0.f;
    const float gadt = p.g_adt ? p.g_adt[(size_t)row * H + h] : 0.f;
    dst[o_dt + h] = dt_pass ? fmaf(-a_mag, gadt, gdt) * sigmoidf_acc(u) : 0.f;
    dst[o_dt + H + h] = a_pass ? -dtv * gadt * sigmoidf_acc(ar) : 0.f;
  }
}

// d dt_bias[h] = sum over rows of the dt column h of d_projected: thread i
// adds rows i, i + 256, ... in order, then a fixed pairwise tree.
__global__ __launch_bounds__(256) void preprocess_bwd_bias_kernel(PreBwdK p) {
  __shared__ float part[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int col = 2 * p.I + 2 * p.M + h;
  float s = 0.f;
  for (int r = tid; r < p.rows; r += blockDim.x) s += p.d_projected[(size_t)r * p.W + col];
  part[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) p.d_dt_bias[h] = part[0];
}

}  // namespace

hipError_t launch_preprocess_bwd(const PreGeom& g, const PreBwdOperands& o, hipStream_t stream) {
  PreBwdK k{};
  k.projected = o.projected; k.dt_bias = o.dt_bias;
  k.g_x = o.g_x; k.g_z = o.g_z; k.g_bh = o.g_bh; k.g_ch = o.g_ch; k.g_dt = o.g_dt; k.g_adt = o.g_adt;
  k.g_trap = o.g_trap; k.g_angle = o.g_angle;
  k.d_projected = o.d_projected; k.d_dt_bias = o.d_dt_bias;
  k.M = (int)(g.G * g.R * g.N);
  k.rows = (int)g.rows; k.I = (int)g.I; k.N = (int)g.N; k.H = (int)g.H; k.A = (int)g.A;
  k.W = 2 * k.I + 2 * k.M + 3 * k.H + k.A;
  k.eps = g.eps; k.dt_min = g.dt_min; k.dt_max = g.dt_max; k.a_floor = g.a_floor;
  hipLaunchKernelGGL(preprocess_bwd_kernel, dim3(g.rows), dim3(256), 0, stream, k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(preprocess_bwd_bias_kernel, dim3(g.H), dim3(256), 0, stream, k);
  return hipGetLastError();
}

}  // namespace m3
