// One Mamba-3 SISO decode token for gfx950: mamba3_siso_step of the oarust
// 0.8.6 page src/rs/ml/matrix/mamba3.rs (state layouts SSM [B,H,P,N],
// cumulative angle [B,H,A], previous key [B,H,N], previous value [B,H,P];
// dispatch_mamba3_siso_step for the shape rules).
//
// Per (batch, head), one workgroup:
//   theta = angle_state + dt * angle;  K = rot(B + b_bias, theta);
//   Q = rot(C + c_bias, theta);  a = exp(adt);  lam = sigmoid(trap);
//   h = a h + (1-lam) dt a v_state k_state^T + lam dt x K^T   (in place)
//   y = h Q (+ D x) (* silu z);  angle_state = theta;  k_state = K;  v_state = x
// The state is streamed once: each row of h is read, updated, written back
// and reduced against Q by a group of lanes.  The kernel is bound by HBM.
#include "common.h"
#include "launch.h"

namespace m3 {
namespace {

struct StepKParams {
  const float *c, *b, *x, *z, *adt, *dt, *trap, *angle, *c_bias, *b_bias, *d;
  float* out;
  float *ssm, *ang_state, *k_state, *v_state;
  int B, H, G, P, N, A;
  int has_z, has_d;
  int sg;        // lanes per state row (power of two <= 64)
  int log2_sg;
};

// LDS: K[N], Q[N], kprev[N], vprev[P], x[P], y[P]
template <int VEC>
__global__ __launch_bounds__(256) void siso_step_kernel(StepKParams p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int g = h / (p.H / p.G);
  const int N = p.N, P = p.P, A = p.A;
  float* Kv = lds;
  float* Qv = Kv + N;
  float* kp = Qv + N;
  float* vp = kp + N;
  float* xv = vp + P;
  float* yv = xv + P;

  const size_t sidx = (size_t)b * p.H + h;  // scalar index for [B,1,H]
  const float dtv = p.dt[sidx];
  const float alpha = expf(p.adt[sidx]);
  const float lam = sigmoidf_acc(p.trap[sidx]);
  const float gam = lam * dtv;
  const float beta = (1.f - lam) * dtv * alpha;

  // Old previous key / value and the new x into LDS before anything is written.
  for (int i = tid; i < N; i += nthreads) kp[i] = p.k_state[sidx * N + i];
  for (int i = tid; i < P; i += nthreads) {
    vp[i] = p.v_state[sidx * P + i];
    xv[i] = p.x[sidx * P + i];
  }
  // Rotated key and query for this token.
  const size_t row = ((size_t)b * p.G + g) * N;
  const size_t brow = (size_t)h * N;
  for (int j = tid; j < N - A; j += nthreads) {
    if (j < A) {
      // theta exact in float64 (the stored state is its float32 rounding)
      const double th = fma((double)dtv, (double)p.angle[(size_t)b * A + j], (double)p.ang_state[sidx * A + j]);
      float s, co;
      sincos_acc_d(th, &s, &co);
      const float b0 = p.b[row + j] + p.b_bias[brow + j];
      const float b1 = p.b[row + j + A] + p.b_bias[brow + j + A];
      const float c0 = p.c[row + j] + p.c_bias[brow + j];
      const float c1 = p.c[row + j + A] + p.c_bias[brow + j + A];
      Kv[j] = b0 * co - b1 * s;
      Kv[j + A] = b0 * s + b1 * co;
      Qv[j] = c0 * co - c1 * s;
      Qv[j + A] = c0 * s + c1 * co;
    } else {
      const int n = j + A;
      Kv[n] = p.b[row + n] + p.b_bias[brow + n];
      Qv[n] = p.c[row + n] + p.c_bias[brow + n];
    }
  }
  __syncthreads();

  // Stream the state: a group of sg lanes owns one row p at a time.
  const int lane = tid & 63;
  const int sg = p.sg;
  const int sl = lane & (sg - 1);
  const int groups_per_wave = 64 >> p.log2_sg;
  const int grp = (tid >> 6) * groups_per_wave + (lane >> p.log2_sg);
  const int ngroups = (nthreads >> 6) * groups_per_wave;
  const int NV = N / VEC;
  float* st = p.ssm + sidx * (size_t)P * N;
  for (int pr = grp; pr < P; pr += ngroups) {
    const float cx = gam * xv[pr];
    const float cv = beta * vp[pr];
    float acc = 0.f;
    float* rowp = st + (size_t)pr * N;
    for (int v = sl; v < NV; v += sg) {
      if constexpr (VEC == 4) {
        floatx4 hv = *reinterpret_cast<const floatx4*>(rowp + 4 * v);
        const floatx4 kk = *reinterpret_cast<const floatx4*>(kp + 4 * v);
        const floatx4 KK = *reinterpret_cast<const floatx4*>(Kv + 4 * v);
        const floatx4 qq = *reinterpret_cast<const floatx4*>(Qv + 4 * v);
        hv.x = fmaf(cx, KK.x, fmaf(cv, kk.x, alpha * hv.x));
        hv.y = fmaf(cx, KK.y, fmaf(cv, kk.y, alpha * hv.y));
        hv.z = fmaf(cx, KK.z, fmaf(cv, kk.z, alpha * hv.z));
        hv.w = fmaf(cx, KK.w, fmaf(cv, kk.w, alpha * hv.w));
        *reinterpret_cast<floatx4*>(rowp + 4 * v) = hv;
        acc = fmaf(hv.x, qq.x, acc);
        acc = fmaf(hv.y, qq.y, acc);
        acc = fmaf(hv.z, qq.z, acc);
        acc = fmaf(hv.w, qq.w, acc);
      } else {
        float hv = rowp[v];
        hv = fmaf(cx, Kv[v], fmaf(cv, kp[v], alpha * hv));
        rowp[v] = hv;
        acc = fmaf(hv, Qv[v], acc);
      }
    }
    for (int off = sg >> 1; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (sl == 0) yv[pr] = acc;
  }
  __syncthreads();

  // Output and the three small states.
  const float dh = p.has_d ? p.d[h] : 0.f;
  for (int i = tid; i < P; i += nthreads) {
    float y = yv[i];
    if (p.has_d) y = fmaf(dh, xv[i], y);
    if (p.has_z) y *= siluf_acc(p.z[sidx * P + i]);
    p.out[sidx * P + i] = y;
    p.v_state[sidx * P + i] = xv[i];
  }
  for (int i = tid; i < N; i += nthreads) p.k_state[sidx * N + i] = Kv[i];
  for (int a = tid; a < A; a += nthreads)
    p.ang_state[sidx * A + a] = fmaf(dtv, p.angle[(size_t)b * A + a], p.ang_state[sidx * A + a]);
}

// N = 128, P = 64 with a 16-byte aligned state: 256 threads per (batch,
// head).  Wave w, pass i covers state rows 8 i + 2 w (lanes 0-31) and
// 8 i + 2 w + 1 (lanes 32-63), one 16-byte item per lane, so each load or
// store instruction moves 1 KiB of contiguous state.  All eight passes are
// loaded before anything else happens, so one memory round trip covers the
// whole 32 KiB state; the row sums of h Q are 32-lane DPP reductions.
__global__ __launch_bounds__(256) void siso_step_n128p64_kernel(StepKParams p) {
  constexpr int N = 128, P = 64;
  __shared__ __attribute__((aligned(16))) float Kv[N];
  __shared__ __attribute__((aligned(16))) float Qv[N];
  __shared__ __attribute__((aligned(16))) float kp[N];
  __shared__ float vp[P], xv[P], yv[P];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int bh = blockIdx.x;
  const int b = bh / p.H;
  const int h = bh - b * p.H;
  const int g = h / (p.H / p.G);
  const int A = p.A;
  const size_t sidx = (size_t)bh;  // scalar index for [B,1,H]
  float* st = p.ssm + sidx * (size_t)P * N;
  const int c4 = 4 * (lane & 31);  // this lane's four state columns
  const int r0 = 2 * wave + (lane >> 5);  // row of pass 0; pass i adds 8 i
  floatx4 hv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) hv[i] = *reinterpret_cast<const floatx4*>(st + (size_t)(r0 + 8 * i) * N + c4);

  const float dtv = p.dt[sidx];
  const float alpha = expf(p.adt[sidx]);
  const float lam = sigmoidf_acc(p.trap[sidx]);
  const float gam = lam * dtv;
  const float beta = (1.f - lam) * dtv * alpha;
  // old previous key / value, the new x, and the rotated key and query
  if (tid < N) kp[tid] = p.k_state[sidx * N + tid];
  if (tid < P) {
    vp[tid] = p.v_state[sidx * P + tid];
    xv[tid] = p.x[sidx * P + tid];
  }
  const size_t row = ((size_t)b * p.G + g) * N;
  const size_t brow = (size_t)h * N;
  if (tid < N - A) {
    const int j = tid;
    if (j < A) {
      // theta exact in float64 (the stored state is its float32 rounding)
      const double th = fma((double)dtv, (double)p.angle[(size_t)b * A + j], (double)p.ang_state[sidx * A + j]);
      float s, co;
      sincos_acc_d(th, &s, &co);
      const float b0 = p.b[row + j] + p.b_bias[brow + j];
      const float b1 = p.b[row + j + A] + p.b_bias[brow + j + A];
      const float c0 = p.c[row + j] + p.c_bias[brow + j];
      const float c1 = p.c[row + j + A] + p.c_bias[brow + j + A];
      Kv[j] = b0 * co - b1 * s;
      Kv[j + A] = b0 * s + b1 * co;
      Qv[j] = c0 * co - c1 * s;
      Qv[j + A] = c0 * s + c1 * co;
    } else {
      const int n = j + A;
      Kv[n] = p.b[row + n] + p.b_bias[brow + n];
      Qv[n] = p.c[row + n] + p.c_bias[brow + n];
    }
  }
  __syncthreads();

  const floatx4 KK = *reinterpret_cast<const floatx4*>(Kv + c4);
  const floatx4 QQ = *reinterpret_cast<const floatx4*>(Qv + c4);
  const floatx4 kk = *reinterpret_cast<const floatx4*>(kp + c4);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = r0 + 8 * i;
    const float cx = gam * xv[r];
    const float cv = beta * vp[r];
    floatx4 v = hv[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = fmaf(cx, KK[e], fmaf(cv, kk[e], alpha * v[e]));
    *reinterpret_cast<floatx4*>(st + (size_t)r * N + c4) = v;
    float acc = v[0] * QQ[0];
    acc = fmaf(v[1], QQ[1], acc);
    acc = fmaf(v[2], QQ[2], acc);
    acc = fmaf(v[3], QQ[3], acc);
    acc = scan32_f(acc);  // lane 31 / 63 hold the row sums
    if ((lane & 31) == 31) yv[r] = acc;
  }
  __syncthreads();

  const float dh = p.has_d ? p.d[h] : 0.f;
  if (tid < P) {
    float y = yv[tid];
    if (p.has_d) y = fmaf(dh, xv[tid], y);
    if (p.has_z) y *= siluf_acc(p.z[sidx * P + tid]);
    p.out[sidx * P + tid] = y;
    p.v_state[sidx * P + tid] = xv[tid];
  }
  if (tid < N) p.k_state[sidx * N + tid] = Kv[tid];
  if (tid < A) p.ang_state[sidx * A + tid] = fmaf(dtv, p.angle[(size_t)b * A + tid], p.ang_state[sidx * A + tid]);
}

}  // namespace

hipError_t launch_siso_step(const ScanGeom& g, const ScanOperands& o, const StepStates& s,
                            hipStream_t stream) {
  StepKParams kp{};
  kp.c = o.c; kp.b = o.b; kp.x = o.x; kp.z = o.z; kp.adt = o.adt; kp.dt = o.dt; kp.trap = o.trap;
  kp.angle = o.angle; kp.c_bias = o.c_bias; kp.b_bias = o.b_bias; kp.d = o.d; kp.out = o.out;
  kp.ssm = s.ssm; kp.ang_state = s.angle; kp.k_state = s.k; kp.v_state = s.v;
  kp.B = g.B; kp.H = g.H; kp.G = g.G; kp.P = g.P; kp.N = g.N; kp.A = g.A;
  kp.has_z = g.has_z; kp.has_d = g.has_d;
  const bool vec4 = (g.N % 4u) == 0u && (reinterpret_cast<uintptr_t>(s.ssm) % 16u) == 0u;
  if (vec4 && g.N == 128 && g.P == 64) {
    hipLaunchKernelGGL(siso_step_n128p64_kernel, dim3(g.B * g.H), dim3(256), 0, stream, kp);
    return hipGetLastError();
  }
  const int NV = vec4 ? (int)g.N / 4 : (int)g.N;
  int sg = 1, lg = 0;
  while (sg < NV && sg < 64) { sg <<= 1; ++lg; }
  kp.sg = sg;
  kp.log2_sg = lg;
  const size_t lds = (size_t)(3 * g.N + 3 * g.P) * sizeof(float) + 16;
  const unsigned grid = g.B * g.H;
  if (vec4)
    hipLaunchKernelGGL(siso_step_kernel<4>, dim3(grid), dim3(256), lds, stream, kp);
  else
    hipLaunchKernelGGL(siso_step_kernel<1>, dim3(grid), dim3(256), lds, stream, kp);
  return hipGetLastError();
}

}  // namespace m3
