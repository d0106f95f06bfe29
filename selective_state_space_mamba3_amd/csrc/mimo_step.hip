// One Mamba-3 MIMO decode token for gfx950: mamba3_mimo_step of the oarust
// 0.8.6 page src/rs/ml/matrix/mamba3.rs (dispatch_mamba3_mimo_step for the
// four state layouts: SSM [B,H,P,N], cumulative angle [B,H,A], previous keys
// [B,H,R,N], previous values [B,H,R,P]; MimoGeometry for the operands).
//
// Per (batch, head), one workgroup:
//   theta = angle_state + dt * angle;  X_r = x * mimo_x[h,r];
//   K_r = rot(B_r + b_bias[h,r], theta);  Q_r = rot(C_r + c_bias[h,r], theta);
//   h = a h + (1-lam) dt a sum_r v_state_r k_state_r^T + lam dt sum_r X_r K_r^T
//   Y_r = (h Q_r + D X_r) * silu(z * mimo_z[h,r]), RMS-normalised over P
//         (eps 1e-5) times norm_weight[h] when has_output_norm;
//   out = sum_r mimo_o[h,r] * Y_r;  angle_state = theta;  k_state_r = K_r;
//   v_state_r = X_r.
// The state is streamed once; the kernel is bound by HBM.
#include "common.h"
#include "launch.h"

namespace m3 {
namespace {

constexpr float kMimoNormEps = 1.0e-5f;  // the MIMO output-norm epsilon of the MIMO push constants

struct MimoStepParams {
  const float *c, *b, *x, *z, *adt, *dt, *trap, *angle, *c_bias, *b_bias, *d;
  const float *mimo_x, *mimo_z, *mimo_o, *norm_weight;
  float* out;
  float *ssm, *ang_state, *k_state, *v_state;
  int B, H, G, P, N, A, R;
  int has_z, has_d, has_norm;
};

// Shared set-up of both kernels: scalars, and in LDS the old previous keys
// and values (kp [R][N], vp [R][P]), X_r (xr [R][P]) and the new rotated
// keys and queries (Kv, Qv [R][N]).  The caller synchronises afterwards.
struct StepScalars {
  float dtv, alpha, gam, beta;
};

__device__ __forceinline__ StepScalars mimo_step_setup(const MimoStepParams& p, int bh, float* Kv, float* Qv,
                                                       float* kp, float* vp, float* xr, int tid, int nthreads) {
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int g = h / (p.H / p.G);
  const int N = p.N, P = p.P, A = p.A, R = p.R;
  StepScalars s;
  s.dtv = p.dt[bh];
  s.alpha = expf(p.adt[bh]);
  const float lam = sigmoidf_acc(p.trap[bh]);
  s.gam = lam * s.dtv;
  s.beta = (1.f - lam) * s.dtv * s.alpha;
  for (int i = tid; i < R * N; i += nthreads) kp[i] = p.k_state[(size_t)bh * R * N + i];
  for (int i = tid; i < R * P; i += nthreads) {
    const int r = i / P, pp = i - r * P;
    vp[i] = p.v_state[(size_t)bh * R * P + i];
    xr[i] = p.x[(size_t)bh * P + pp] * p.mimo_x[((size_t)h * R + r) * P + pp];
  }
  // column j < A: the pair (j, j + A); A <= j < N - A: the plain column j + A
  for (int j = tid; j < N - A; j += nthreads) {
    float sn = 0.f, co = 1.f;
    // theta exact in float64 (the stored state is its float32 rounding)
    if (j < A)
      sincos_acc_d(fma((double)s.dtv, (double)p.angle[(size_t)b * A + j], (double)p.ang_state[(size_t)bh * A + j]),
                   &sn, &co);
    for (int r = 0; r < R; ++r) {
      const float* brow = p.b + ((size_t)b * R * p.G + (size_t)r * p.G + g) * N;
      const float* crow = p.c + ((size_t)b * R * p.G + (size_t)r * p.G + g) * N;
      const float* bb = p.b_bias + ((size_t)h * R + r) * N;
      const float* cb = p.c_bias + ((size_t)h * R + r) * N;
      float* Kr = Kv + r * N;
      float* Qr = Qv + r * N;
      if (j < A) {
        const float b0 = brow[j] + bb[j], b1 = brow[j + A] + bb[j + A];
        const float c0 = crow[j] + cb[j], c1 = crow[j + A] + cb[j + A];
        Kr[j] = b0 * co - b1 * sn;
        Kr[j + A] = b0 * sn + b1 * co;
        Qr[j] = c0 * co - c1 * sn;
        Qr[j + A] = c0 * sn + c1 * co;
      } else {
        const int n = j + A;
        Kr[n] = brow[n] + bb[n];
        Qr[n] = crow[n] + cb[n];
      }
    }
  }
  return s;
}

// Epilogue and the small-state updates once yv [R][P] holds h Q_r.
// Wave w handles ranks w, w + nwaves, ...; each lane two head_dim items.
__device__ __forceinline__ void mimo_step_finish(const MimoStepParams& p, int bh, const StepScalars& s,
                                                 const float* Kv, const float* xr, float* yv,
                                                 int tid, int nthreads) {
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int N = p.N, P = p.P, A = p.A, R = p.R;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthreads >> 6;
  const float dh = p.has_d ? p.d[h] : 0.f;
  for (int r = wave; r < R; r += nwaves) {
    float yy[2];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pp = lane + 64 * k;
      float y = 0.f;
      if (pp < P) {
        y = yv[r * P + pp];
        if (p.has_d) y = fmaf(dh, xr[r * P + pp], y);
        if (p.has_z) y *= siluf_acc(p.z[(size_t)bh * P + pp] * p.mimo_z[((size_t)h * R + r) * P + pp]);
      }
      yy[k] = y;
      ss = fmaf(y, y, ss);
    }
    float inv = 1.f;
    if (p.has_norm) inv = 1.f / sqrtf(read_lane_f(scan64_f(ss), 63) / (float)P + kMimoNormEps);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pp = lane + 64 * k;
      if (pp < P) {
        float y = yy[k];
        if (p.has_norm) y = y * inv * p.norm_weight[(size_t)h * P + pp];
        yv[r * P + pp] = y * p.mimo_o[((size_t)h * R + r) * P + pp];
      }
    }
  }
  __syncthreads();
  for (int pp = tid; pp < P; pp += nthreads) {
    float o = 0.f;
    for (int r = 0; r < R; ++r) o += yv[r * P + pp];
    p.out[(size_t)bh * P + pp] = o;
  }
  for (int i = tid; i < R * P; i += nthreads) p.v_state[(size_t)bh * R * P + i] = xr[i];
  for (int i = tid; i < R * N; i += nthreads) p.k_state[(size_t)bh * R * N + i] = Kv[i];
  for (int a = tid; a < A; a += nthreads)
    p.ang_state[(size_t)bh * A + a] = fmaf(s.dtv, p.angle[(size_t)b * A + a], p.ang_state[(size_t)bh * A + a]);
}

// N = 128, P = 64, 16-byte aligned state, rank R fixed at compile time:
// 256 threads per (batch, head).  Wave w, pass i covers state rows 8 i + 2 w
// (lanes 0-31) and 8 i + 2 w + 1 (lanes 32-63), one 16-byte item per lane,
// so each load or store moves 1 KiB of contiguous state.  Every global load
// of the workgroup (the eight state items, the set-up operands and the
// epilogue operands) is issued before the first one is used, so one memory
// round trip covers them all; the loads use clamped in-range indices rather
// than branches.  A lane's key and query columns are the same in all eight
// passes, so for R <= 4 they are held in registers.
template <int R>
__global__ __launch_bounds__(256) void mimo_step_n128p64_kernel(MimoStepParams p) {
  constexpr int N = 128, P = 64;
  constexpr bool HOIST = R <= 4;
  constexpr int KPN = (R * N + 255) / 256;  // previous-key items per thread
  constexpr int VPN = (R * P + 255) / 256;  // previous-value / X_r items per thread
  constexpr int KR = (R + 3) / 4;           // epilogue ranks per wave
  __shared__ __attribute__((aligned(16))) float Kv[R * N];
  __shared__ __attribute__((aligned(16))) float Qv[R * N];
  __shared__ __attribute__((aligned(16))) float kp[R * N];
  __shared__ float vp[R * P], xr[R * P], yv[R * P];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int g = h / (p.H / p.G);
  const int A = p.A;
  float* st = p.ssm + (size_t)bh * P * N;
  const int c4 = 4 * (lane & 31);
  const int r0 = 2 * wave + (lane >> 5);

  floatx4 hv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) hv[i] = *reinterpret_cast<const floatx4*>(st + (size_t)(r0 + 8 * i) * N + c4);

  // set-up operands
  const float dtv = p.dt[bh];
  const float adtv = p.adt[bh];
  const float trv = p.trap[bh];
  const float dh = p.has_d ? p.d[h] : 0.f;
  float kpl[KPN], vpl[VPN], xl[VPN], mxl[VPN];
#pragma unroll
  for (int k = 0; k < KPN; ++k) kpl[k] = p.k_state[(size_t)bh * R * N + min(tid + 256 * k, R * N - 1)];
#pragma unroll
  for (int k = 0; k < VPN; ++k) {
    const int i = min(tid + 256 * k, R * P - 1);
    vpl[k] = p.v_state[(size_t)bh * R * P + i];
    xl[k] = p.x[(size_t)bh * P + (i & (P - 1))];
    mxl[k] = p.mimo_x[(size_t)h * R * P + i];
  }
  // column j < A: the pair (j, j + A); A <= j < N - A: the plain column j + A
  const int j = min(tid, N - A - 1);
  const int n0 = j < A ? j : j + A;
  const int n1 = j < A ? j + A : n0;
  float bl0[R], bl1[R], bb0[R], bb1[R], cl0[R], cl1[R], cb0[R], cb1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* brow = p.b + ((size_t)b * R * p.G + (size_t)r * p.G + g) * N;
    const float* crow = p.c + ((size_t)b * R * p.G + (size_t)r * p.G + g) * N;
    const float* bb = p.b_bias + ((size_t)h * R + r) * N;
    const float* cb = p.c_bias + ((size_t)h * R + r) * N;
    bl0[r] = brow[n0]; bl1[r] = brow[n1]; bb0[r] = bb[n0]; bb1[r] = bb[n1];
    cl0[r] = crow[n0]; cl1[r] = crow[n1]; cb0[r] = cb[n0]; cb1[r] = cb[n1];
  }
  float ang = 0.f, ast = 0.f;
  if (A > 0) {
    const int ja = min(j, A - 1);
    ang = p.angle[(size_t)b * A + ja];
    ast = p.ang_state[(size_t)bh * A + ja];
  }
  // epilogue operands of this wave's ranks (wave, wave + 4)
  const float* zp = p.has_z ? p.z : p.x;
  const float* mzp = p.has_z ? p.mimo_z : p.mimo_o;
  const float* nwp = p.has_norm ? p.norm_weight : p.mimo_o;
  const float zl = zp[(size_t)bh * P + lane];
  const float nwl = nwp[(size_t)h * P + lane];
  float mzl[KR], mol[KR];
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int r = min(wave + 4 * k, R - 1);
    mzl[k] = mzp[((size_t)h * R + r) * P + lane];
    mol[k] = p.mimo_o[((size_t)h * R + r) * P + lane];
  }

  // scalars and the set-up into LDS
  const float alpha = expf(adtv);
  const float lam = sigmoidf_acc(trv);
  const float gam = lam * dtv;
  const float beta = (1.f - lam) * dtv * alpha;
#pragma unroll
  for (int k = 0; k < KPN; ++k)
    if (tid + 256 * k < R * N) kp[tid + 256 * k] = kpl[k];
#pragma unroll
  for (int k = 0; k < VPN; ++k)
    if (tid + 256 * k < R * P) {
      vp[tid + 256 * k] = vpl[k];
      xr[tid + 256 * k] = xl[k] * mxl[k];
    }
  const float th = fmaf(dtv, ang, ast);  // the stored state: float32 rounding of the exact theta
  if (tid < N - A) {
    if (j < A) {
      float sn, co;
      sincos_acc_d(fma((double)dtv, (double)ang, (double)ast), &sn, &co);  // theta exact in float64
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float k0 = bl0[r] + bb0[r], k1 = bl1[r] + bb1[r];
        const float q0 = cl0[r] + cb0[r], q1 = cl1[r] + cb1[r];
        Kv[r * N + j] = k0 * co - k1 * sn;
        Kv[r * N + j + A] = k0 * sn + k1 * co;
        Qv[r * N + j] = q0 * co - q1 * sn;
        Qv[r * N + j + A] = q0 * sn + q1 * co;
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        Kv[r * N + n0] = bl0[r] + bb0[r];
        Qv[r * N + n0] = cl0[r] + cb0[r];
      }
    }
  }
  __syncthreads();

  // the new small states (every read of the old ones is done)
  if (tid < A) p.ang_state[(size_t)bh * A + tid] = th;
#pragma unroll
  for (int k = 0; k < KPN; ++k)
    if (tid + 256 * k < R * N) p.k_state[(size_t)bh * R * N + tid + 256 * k] = Kv[tid + 256 * k];
#pragma unroll
  for (int k = 0; k < VPN; ++k)
    if (tid + 256 * k < R * P) p.v_state[(size_t)bh * R * P + tid + 256 * k] = xr[tid + 256 * k];

  floatx4 kkr[HOIST ? R : 1], KKr[HOIST ? R : 1], QQr[HOIST ? R : 1];
  if constexpr (HOIST) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      kkr[r] = *reinterpret_cast<const floatx4*>(kp + r * N + c4);
      KKr[r] = *reinterpret_cast<const floatx4*>(Kv + r * N + c4);
      QQr[r] = *reinterpret_cast<const floatx4*>(Qv + r * N + c4);
    }
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r0 + 8 * i;
    floatx4 v = hv[i] * alpha;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const floatx4 kk = HOIST ? kkr[r] : *reinterpret_cast<const floatx4*>(kp + r * N + c4);
      const floatx4 KK = HOIST ? KKr[r] : *reinterpret_cast<const floatx4*>(Kv + r * N + c4);
      const float cv = beta * vp[r * P + row];
      const float cx = gam * xr[r * P + row];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = fmaf(cx, KK[e], fmaf(cv, kk[e], v[e]));
    }
    *reinterpret_cast<floatx4*>(st + (size_t)row * N + c4) = v;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const floatx4 QQ = HOIST ? QQr[r] : *reinterpret_cast<const floatx4*>(Qv + r * N + c4);
      float a = v[0] * QQ[0];
      a = fmaf(v[1], QQ[1], a);
      a = fmaf(v[2], QQ[2], a);
      acc[r] = fmaf(v[3], QQ[3], a);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = scan32_f(acc[r]);  // lane 31 / 63 hold the row sums
    if ((lane & 31) == 31) {
#pragma unroll
      for (int r = 0; r < R; ++r) yv[r * P + row] = acc[r];
    }
  }
  __syncthreads();

  // epilogue: wave w handles ranks w and w + 4, lane = head_dim index
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int r = wave + 4 * k;
    if (r < R) {
      float y = yv[r * P + lane];
      if (p.has_d) y = fmaf(dh, xr[r * P + lane], y);
      if (p.has_z) y *= siluf_acc(zl * mzl[k]);
      if (p.has_norm) {
        const float ss = read_lane_f(scan64_f(y * y), 63);
        y = y * (1.f / sqrtf(ss / (float)P + kMimoNormEps)) * nwl;
      }
      yv[r * P + lane] = y * mol[k];
    }
  }
  __syncthreads();
  if (tid < P) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) o += yv[r * P + tid];
    p.out[(size_t)bh * P + tid] = o;
  }
}

// Any N, P (<= 128), R <= 8: a group of sg lanes owns one state row at a
// time, each lane striding over its columns.  LDS: Kv, Qv, kp [R][N];
// vp, xr, yv [R][P].
__global__ __launch_bounds__(256) void mimo_step_kernel(MimoStepParams p, int sg, int log2_sg) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int bh = blockIdx.x;
  const int N = p.N, P = p.P, R = p.R;
  float* Kv = lds;
  float* Qv = Kv + R * N;
  float* kp = Qv + R * N;
  float* vp = kp + R * N;
  float* xr = vp + R * P;
  float* yv = xr + R * P;
  const StepScalars s = mimo_step_setup(p, bh, Kv, Qv, kp, vp, xr, tid, nthreads);
  __syncthreads();

  const int lane = tid & 63;
  const int sl = lane & (sg - 1);
  const int groups_per_wave = 64 >> log2_sg;
  const int grp = (tid >> 6) * groups_per_wave + (lane >> log2_sg);
  const int ngroups = (nthreads >> 6) * groups_per_wave;
  float* st = p.ssm + (size_t)bh * P * N;
  for (int pr = grp; pr < P; pr += ngroups) {
    float* rowp = st + (size_t)pr * N;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int n = sl; n < N; n += sg) {
      float hv = rowp[n] * s.alpha;
      for (int r = 0; r < R; ++r)
        hv = fmaf(s.gam * xr[r * P + pr], Kv[r * N + n], fmaf(s.beta * vp[r * P + pr], kp[r * N + n], hv));
      rowp[n] = hv;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (r < R) acc[r] = fmaf(hv, Qv[r * N + n], acc[r]);
    }
    for (int r = 0; r < R; ++r) {
      float a = acc[r];
      for (int off = sg >> 1; off > 0; off >>= 1) a += __shfl_xor(a, off, 64);
      if (sl == 0) yv[r * P + pr] = a;
    }
  }
  __syncthreads();
  mimo_step_finish(p, bh, s, Kv, xr, yv, tid, nthreads);
}

}  // namespace

hipError_t launch_mimo_step(const ScanGeom& g, const ScanOperands& o, const StepStates& s,
                            hipStream_t stream) {
  MimoStepParams kp{};
  kp.c = o.c; kp.b = o.b; kp.x = o.x; kp.z = o.z; kp.adt = o.adt; kp.dt = o.dt; kp.trap = o.trap;
  kp.angle = o.angle; kp.c_bias = o.c_bias; kp.b_bias = o.b_bias; kp.d = o.d;
  kp.mimo_x = o.mimo_x; kp.mimo_z = o.mimo_z; kp.mimo_o = o.mimo_o; kp.norm_weight = o.norm_weight;
  kp.out = o.out;
  kp.ssm = s.ssm; kp.ang_state = s.angle; kp.k_state = s.k; kp.v_state = s.v;
  kp.B = g.B; kp.H = g.H; kp.G = g.G; kp.P = g.P; kp.N = g.N; kp.A = g.A; kp.R = g.R;
  kp.has_z = g.has_z; kp.has_d = g.has_d; kp.has_norm = g.has_norm;
  const unsigned grid = g.B * g.H;
  const bool al16 = (reinterpret_cast<uintptr_t>(s.ssm) % 16u) == 0u;
  if (al16 && g.N == 128 && g.P == 64 && g.R >= 1 && g.R <= 8) {
    switch (g.R) {
      case 1: hipLaunchKernelGGL(mimo_step_n128p64_kernel<1>, dim3(grid), dim3(256), 0, stream, kp); break;
      case 2: hipLaunchKernelGGL(mimo_step_n128p64_kernel<2>, dim3(grid), dim3(256), 0, stream, kp); break;
      case 3: hipLaunchKernelGGL(mimo_step_n128p64_kernel<3>, dim3(grid), dim3(256), 0, stream, kp); break;
      case 4: hipLaunchKernelGGL(mimo_step_n128p64_kernel<4>, dim3(grid), dim3(256), 0, stream, kp); break;
      case 5: hipLaunchKernelGGL(mimo_step_n128p64_kernel<5>, dim3(grid), dim3(256), 0, stream, kp); break;
      case 6: hipLaunchKernelGGL(mimo_step_n128p64_kernel<6>, dim3(grid), dim3(256), 0, stream, kp); break;
      case 7: hipLaunchKernelGGL(mimo_step_n128p64_kernel<7>, dim3(grid), dim3(256), 0, stream, kp); break;
      default: hipLaunchKernelGGL(mimo_step_n128p64_kernel<8>, dim3(grid), dim3(256), 0, stream, kp); break;
    }
    return hipGetLastError();
  }
  int sg = 1, lg = 0;
  while (sg < (int)g.N && sg < 32) { sg <<= 1; ++lg; }
  const size_t lds = (size_t)(3 * g.R * g.N + 3 * g.R * g.P) * sizeof(float);
  hipLaunchKernelGGL(mimo_step_kernel, dim3(grid), dim3(256), lds, stream, kp, sg, lg);
  return hipGetLastError();
}

}  // namespace m3
