// Fused Mamba-3 projection preprocess for gfx950: mamba3_preprocess of the
// oarust 0.8.6 page src/rs/ml/matrix/mamba3.rs (Mamba3PreprocessConfig,
// Mamba3PreprocessResult, PreprocessGeometry; packed width
// 2I + 2GRN + 3H + A).
//
// Columns of a packed row, in the order the dispatch binds its outputs:
//   z [I] | x [I] | B [G*R*N] | C [G*R*N] | dt_raw [H] | A_raw [H] | trap [H] | angle [A]
// Outputs: x, z, trap, angle copied; each N-wide B and C row scaled by
// 1/sqrt(mean(v^2) + eps); dt = clamp(softplus(dt_raw + dt_bias), dt_min,
// dt_max); adt = -max(softplus(A_raw), a_floor) * dt.
//
// One workgroup per packed row (several rows per workgroup for narrow
// rows); every byte is read once and written once, so the kernel is bound
// by HBM.  Copies use 16-byte accesses when the row width and the slice
// widths keep them aligned.
#include "common.h"
#include "launch.h"

namespace m3 {
namespace {

struct PreKParams {
  const float *projected, *dt_bias;
  float *x, *z, *bh, *ch, *dt, *adt, *trap, *angle;
  int rows, W, I, N, H, A, M;  // M = G*R*N
  float eps, dt_min, dt_max, a_floor;
};

__device__ __forceinline__ void copy_slice(const float* __restrict__ src, float* __restrict__ dst,
                                           int n, int tid, int nthreads, bool vec) {
  if (vec) {
    const int n4 = n >> 2;
    for (int i = tid; i < n4; i += nthreads)
      reinterpret_cast<floatx4*>(dst)[i] = reinterpret_cast<const floatx4*>(src)[i];
  } else {
    for (int i = tid; i < n; i += nthreads) dst[i] = src[i];
  }
}

// derived != 0: only bh, ch, dt and adt (the fused preprocess -> scan reads
// x, z, trap and angle straight from the packed rows).
__global__ __launch_bounds__(256) void preprocess_kernel(PreKParams p, int vec, int derived) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = nthreads >> 6;
  const float* row = p.projected + (size_t)r * p.W;
  const bool v = vec != 0;

  if (!derived) {
    copy_slice(row, p.z + (size_t)r * p.I, p.I, tid, nthreads, v);
    copy_slice(row + p.I, p.x + (size_t)r * p.I, p.I, tid, nthreads, v);
  }

  // B and C rows: one wave per N-wide row, lanes over the row.
  const int nrows_bc = 2 * (p.M / p.N);
  for (int j = wave; j < nrows_bc; j += nwaves) {
    const bool is_c = j >= nrows_bc / 2;
    const int k = is_c ? j - nrows_bc / 2 : j;
    const float* src = row + 2 * p.I + (is_c ? p.M : 0) + k * p.N;
    float* dst = (is_c ? p.ch : p.bh) + (size_t)r * p.M + (size_t)k * p.N;
    float ss = 0.f;
    for (int i = lane; i < p.N; i += 64) ss = fmaf(src[i], src[i], ss);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.f / sqrtf(ss / (float)p.N + p.eps);
    for (int i = lane; i < p.N; i += 64) dst[i] = src[i] * inv;
  }

  const float* sc = row + 2 * p.I + 2 * p.M;
  for (int h = tid; h < p.H; h += nthreads) {
    const float dtv = fminf(fmaxf(softplusf_acc(sc[h] + p.dt_bias[h]), p.dt_min), p.dt_max);
    const float amag = fmaxf(softplusf_acc(sc[p.H + h]), p.a_floor);
    p.dt[(size_t)r * p.H + h] = dtv;
    p.adt[(size_t)r * p.H + h] = -amag * dtv;
    if (!derived) p.trap[(size_t)r * p.H + h] = sc[2 * p.H + h];
  }
  if (!derived)
    for (int a = tid; a < p.A; a += nthreads) p.angle[(size_t)r * p.A + a] = sc[3 * p.H + a];
}

// The derived outputs only (bh, ch, dt, adt) for the fused preprocess ->
// scan: one wave per packed row, four rows per workgroup, so the whole grid
// is resident at once.  Each wave loads a B row and the matching C row
// together, then reduces both; lanes h < H take the dt / A columns.
__global__ __launch_bounds__(256) void preprocess_derived_kernel(PreKParams p) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= p.rows) return;
  const float* row = p.projected + (size_t)r * p.W;
  const int nb = p.M / p.N;  // B rows (and C rows) per packed row
  // the dt / A columns of the first 64 heads load with the rows (loaded after
  // the row stores, they were a second round trip)
  const float* sc = row + 2 * p.I + 2 * p.M;
  const bool hv = lane < p.H;
  const float dt_raw = hv ? sc[lane] : 0.f;
  const float a_raw = hv ? sc[p.H + lane] : 0.f;
  const float dt_b = hv ? p.dt_bias[lane] : 0.f;
  for (int k = 0; k < nb; ++k) {
    const float* sb = row + 2 * p.I + k * p.N;
    const float* scc = sb + p.M;
    float vb[2], vc[2], sbs = 0.f, scs = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = lane + 64 * e;
      vb[e] = i < p.N ? sb[i] : 0.f;
      vc[e] = i < p.N ? scc[i] : 0.f;
    }
    // each lane sums its elements in index order, as preprocess_kernel does,
    // so both kernels give the same bits
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      sbs = fmaf(vb[e], vb[e], sbs);
      scs = fmaf(vc[e], vc[e], scs);
    }
    for (int i = lane + 128; i < p.N; i += 64) {  // N > 128: the rest of the sums
      sbs = fmaf(sb[i], sb[i], sbs);
      scs = fmaf(scc[i], scc[i], scs);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      sbs += __shfl_xor(sbs, off, 64);
      scs += __shfl_xor(scs, off, 64);
    }
    const float ib = 1.f / sqrtf(sbs / (float)p.N + p.eps);
    const float ic = 1.f / sqrtf(scs / (float)p.N + p.eps);
    float* db = p.bh + (size_t)r * p.M + (size_t)k * p.N;
    float* dc = p.ch + (size_t)r * p.M + (size_t)k * p.N;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = lane + 64 * e;
      if (i < p.N) {
        db[i] = vb[e] * ib;
        dc[i] = vc[e] * ic;
      }
    }
    for (int i = lane + 128; i < p.N; i += 64) {
      db[i] = sb[i] * ib;
      dc[i] = scc[i] * ic;
    }
  }
  if (hv) {
    const float dtv = fminf(fmaxf(softplusf_acc(dt_raw + dt_b), p.dt_min), p.dt_max);
    const float amag = fmaxf(softplusf_acc(a_raw), p.a_floor);
    p.dt[(size_t)r * p.H + lane] = dtv;
    p.adt[(size_t)r * p.H + lane] = -amag * dtv;
  }
  for (int h = lane + 64; h < p.H; h += 64) {
    const float dtv = fminf(fmaxf(softplusf_acc(sc[h] + p.dt_bias[h]), p.dt_min), p.dt_max);
    const float amag = fmaxf(softplusf_acc(sc[p.H + h]), p.a_floor);
    p.dt[(size_t)r * p.H + h] = dtv;
    p.adt[(size_t)r * p.H + h] = -amag * dtv;
  }
}

}  // namespace

namespace {

hipError_t launch_pre(const PreGeom& g, const PreOperands& o, int derived, hipStream_t stream) {
  PreKParams kp{};
  kp.projected = o.projected; kp.dt_bias = o.dt_bias;
  kp.x = o.x; kp.z = o.z; kp.bh = o.bh; kp.ch = o.ch; kp.dt = o.dt; kp.adt = o.adt;
  kp.trap = o.trap; kp.angle = o.angle;
  kp.rows = (int)g.rows;
  kp.I = (int)g.I; kp.N = (int)g.N; kp.H = (int)g.H; kp.A = (int)g.A;
  kp.M = (int)(g.G * g.R * g.N);
  kp.W = 2 * kp.I + 2 * kp.M + 3 * kp.H + kp.A;
  kp.eps = g.eps; kp.dt_min = g.dt_min; kp.dt_max = g.dt_max; kp.a_floor = g.a_floor;
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) % 16u) == 0u; };
  const int vec = (!derived && kp.W % 4 == 0 && kp.I % 4 == 0 && al16(o.projected) && al16(o.x) && al16(o.z)) ? 1 : 0;
  if (derived)
    hipLaunchKernelGGL(preprocess_derived_kernel, dim3((g.rows + 3) / 4), dim3(256), 0, stream, kp);
  else
    hipLaunchKernelGGL(preprocess_kernel, dim3(g.rows), dim3(256), 0, stream, kp, vec, derived);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_preprocess(const PreGeom& g, const PreOperands& o, hipStream_t stream) {
  return launch_pre(g, o, 0, stream);
}

hipError_t launch_preprocess_derived(const PreGeom& g, const PreOperands& o, hipStream_t stream) {
  return launch_pre(g, o, 1, stream);
}

}  // namespace m3
