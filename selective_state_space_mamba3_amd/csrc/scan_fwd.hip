// Chunked Mamba-3 selective-state scan, forward, for gfx950 (SISO and MIMO).
//
// Operation: mamba3_siso / mamba3_mimo of the oarust 0.8.6 page
// src/rs/ml/matrix/mamba3.rs ("Public API" docs for layouts; Geometry /
// MimoGeometry for the rules).  The per-token recurrence
//     h_t = a_t h_{t-1} + (1-lam_t) dt_t a_t sum_r x_{r,t-1} K_{r,t-1}^T
//           + lam_t dt_t sum_r x_{r,t} K_{r,t}^T,          a_t = exp(adt_t)
// is rewritten with the running state h'_t = h_t + (1-lam_{t+1}) dt_{t+1} u_t
// (u_t the rank sum of x K^T), which obeys h'_t = a_t h'_{t-1} + scale_t u_t
// with scale_t = lam_t dt_t + (1-lam_{t+1}) dt_{t+1}; then
//     y_{r,t} = exp(cum_t) Q_{r,t} h'_entry
//             + sum_{s<t in chunk} exp(cum_t - cum_s) scale_s (Q_{r,t}.K_{r',s}) x_{r',s}
//             + lam_t dt_t sum_{r'} (Q_{r,t}.K_{r',t}) x_{r',t}
// with cum the chunk-local inclusive prefix sum of adt.  These are the
// quantities the SISO backward dispatches name (qk, decay, gamma, scale,
// h_previous), here computed in registers and LDS instead of memory.
//
// Work decomposition
//   * A chunk holds QV = 32 "virtual rows" v = t * RS + r (token t, rank
//     r < R, RS = R rounded up to a power of two so that no token's rows
//     straddle a 16-row MFMA tile; rows with r >= R stay zero).  SISO has
//     R = RS = 1, MIMO stacks its ranks inside the chunk.
//   * One workgroup runs one (batch, head, sequence segment).  Wave w < PT
//     owns the 16 head_dim columns [16w, 16w+16) and keeps the state
//     h'^T [N x 16] of those columns in MFMA accumulator registers for the
//     whole segment; at least four waves share the loads and VALU work.
//   * Intra-chunk S = Q K^T, the decay/trapezoid mask, M X, the carried-state
//     read Q h'^T and the state update K^T (w X) all run on
//     v_mfma_f32_16x16x4_f32.
//   * The next chunk's x, B, C, angle and scalars are loaded into registers
//     while the current chunk's MFMA work runs; z is loaded at the start of
//     the chunk that uses it.  The cumulative angle is a 32-lane scan.
//   * Sequence segments: a first pass computes each segment's end state
//     from a zero entry (plus its decay product and angle increment) into
//     the workspace; the main pass folds the earlier segments' summaries
//     into its entry state, so segments of one sequence run in parallel.
#include "common.h"
#include "launch.h"

#include <stdlib.h>

namespace m3 {
namespace {

constexpr int kAux = 68;        // per segment summary: angle increment [<=64], decay at 64
constexpr int kAuxDecay = 64;
constexpr float kNormEps = 1.0e-5f;  // MIMO output-norm epsilon of the MIMO push constants
constexpr int kQV = 32;         // virtual rows per chunk

struct ScanKParams {
  const float *c, *b, *x, *z, *adt, *dt, *trap, *angle, *c_bias, *b_bias, *d;
  const float *mimo_x, *mimo_z, *mimo_o, *norm_weight;
  float* out;
  float* ws_state;  // [B*H][nseg-1][PT*NT tiles][64 lanes][4]
  float* ws_aux;    // [B*H][nseg-1][kAux]
  int B, L, H, G, P, N, A, R;
  int has_z, has_d, has_norm;
  int NT, PT;       // 16-wide blocks of N and P
  int RS, rs_log2;  // rank stride of the virtual rows (power of two >= R)
  int Qt;           // tokens per chunk (QV / RS)
  int seg_len, nseg;
  // LDS layout (float offsets) and row strides
  int o_ql, o_kl, o_xl, o_ml, o_yl, o_cs, o_bias, o_mimo, o_sc, o_run, lds_floats;
  int ks, xs, ms, ys;
};

template <int VEC>
struct VecOf;
template <>
struct VecOf<4> {
  using T = floatx4;
};
template <>
struct VecOf<1> {
  using T = float;
};

template <int VEC>
__device__ __forceinline__ typename VecOf<VEC>::T vload(const float* p) {
  if constexpr (VEC == 4)
    return *reinterpret_cast<const floatx4*>(p);
  else
    return *p;
}
template <int VEC>
__device__ __forceinline__ void vstore(float* p, const typename VecOf<VEC>::T& v) {
  if constexpr (VEC == 4)
    *reinterpret_cast<floatx4*>(p) = v;
  else
    *p = v;
}
__device__ __forceinline__ float comp(const floatx4& v, int e) { return v[e]; }
__device__ __forceinline__ float comp(const float& v, int) { return v; }
__device__ __forceinline__ void set_comp(floatx4& v, int e, float x) { v[e] = x; }
__device__ __forceinline__ void set_comp(float& v, int, float x) { v = x; }

template <int VEC, bool FULL, bool MIMO>
__global__ __launch_bounds__(512) void scan_chunk_kernel(ScanKParams p) {
  using vec_t = typename VecOf<VEC>::T;
  constexpr int QV = kQV;
  constexpr int TB = QV / 16;
  constexpr int KX = 8 / VEC;   // x / z items per thread (Qt*P/VEC <= 8/VEC * threads)
  constexpr int KB = 16 / VEC;  // B / C row items per thread (QV*N/VEC <= 16/VEC * threads)
  constexpr int KA = 4;         // angle values per lane (launch gives >= A/8 waves)
  constexpr int KZM = 8;        // tokens per wave in the MIMO epilogue
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int nwaves = nthreads >> 6;
  const int l16 = lane & 15;
  const int lq = lane >> 4;

  const int nseg_run = FULL ? p.nseg : p.nseg - 1;
  const uint32_t unit = xcd_remap(blockIdx.x, gridDim.x);
  const int h = unit % p.H;
  const int rest = unit / p.H;
  const int seg = rest % nseg_run;
  const int b = rest / nseg_run;
  const int g = h / (p.H / p.G);
  const int bh = b * p.H + h;
  const int t_begin = seg * p.seg_len;
  const int t_end = min(t_begin + p.seg_len, p.L);
  const int R = p.R;
  const int RG = R * p.G;
  const int Qt = p.Qt;
  const int rsl = p.rs_log2;
  const int N = p.N, P = p.P, A = p.A;
  const int ks = p.ks, xs = p.xs, ms = p.ms, ys = p.ys;
  const bool mma_wave = wave < p.PT;

  float* Ql = lds + p.o_ql;   // [QV][ks] C (+bias), pairs rotated in place   (main pass)
  float* Kl = lds + p.o_kl;   // [QV][ks] B (+bias), pairs rotated in place
  float* Xl = lds + p.o_xl;   // [QV][xs] per-rank x
  float* Ml = lds + p.o_ml;   // [QV][ms] masked S                             (main pass)
  float* Yl = lds + p.o_yl;   // [QV][ys] raw y                                (main pass)
  float* CS = lds + p.o_cs;   // [64] cos / [64] sin for the entry-state fold
  float* SN = CS + 64;
  float* bbL = lds + p.o_bias;  // [R][N] b_bias of this head; cbL follows
  float* cbL = bbL + R * N;
  float* mxL = lds + p.o_mimo;  // [R][P] mimo_x, mimo_z, mimo_o, then norm_weight [P]
  float* mzL = mxL + R * P;
  float* moL = mzL + R * P;
  float* nwL = moL + R * P;
  float* sc_cum = lds + p.o_sc;
  float* sc_ecum = sc_cum + QV;
  float* sc_gam = sc_ecum + QV;
  float* sc_scl = sc_gam + QV;
  float* sc_w = sc_scl + QV;
  float* sc_dt = sc_w + QV;
  float* run = lds + p.o_run;  // [0,64) running theta, [64] chunk decay

  for (int i = tid; i < p.lds_floats; i += nthreads) lds[i] = 0.f;
  __syncthreads();
  for (int i = tid; i < R * N; i += nthreads) {
    bbL[i] = p.b_bias[(size_t)h * R * N + i];
    if (FULL) cbL[i] = p.c_bias[(size_t)h * R * N + i];
  }
  if constexpr (FULL && MIMO) {
    for (int i = tid; i < R * P; i += nthreads) {
      mxL[i] = p.mimo_x[(size_t)h * R * P + i];
      mzL[i] = p.mimo_z[(size_t)h * R * P + i];
      moL[i] = p.mimo_o[(size_t)h * R * P + i];
    }
    for (int i = tid; i < P; i += nthreads) nwL[i] = p.norm_weight[(size_t)h * P + i];
  } else if constexpr (MIMO) {
    for (int i = tid; i < R * P; i += nthreads) mxL[i] = p.mimo_x[(size_t)h * R * P + i];
  }

  const int p0 = wave * 16;
  floatx4 Hacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) Hacc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Entry state: fold the summaries of the earlier segments, in order,
  //   h' <- decay_i h' + rot(theta_i) U_i,
  // where U_i was built with the angle restarted at zero inside segment i, so
  // its state axis is turned by theta_i = the summed angle of the segments
  // before i (the keys it holds are rot(theta_i + local) = rot(theta_i) rot(local)).
  // U_i passes through LDS in [p][n] layout for the pair rotation.
  if (FULL && seg > 0) {
    __syncthreads();
    float* Ub = lds;  // [PT*16][NT*16 + 4], overlays the chunk buffers (unused yet)
    const int us = p.NT * 16 + 4;
    for (int i = 0; i < seg; ++i) {
      const size_t si = (size_t)bh * (p.nseg - 1) + i;
      const float* aux = p.ws_aux + si * kAux;
      const float* st = p.ws_state + si * (size_t)(p.PT * p.NT) * 256;
      if (mma_wave) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          if (nb < p.NT) {
            const floatx4 u = *reinterpret_cast<const floatx4*>(st + ((wave * p.NT + nb) * 64 + lane) * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) Ub[(p0 + l16) * us + nb * 16 + 4 * lq + r] = u[r];
          }
        }
      }
      if (tid < A) {
        float sn, cs;
        sincos_acc(run[tid], &sn, &cs);
        CS[tid] = cs;
        SN[tid] = sn;
      }
      __syncthreads();
      for (int e = tid; e < p.PT * 16 * A; e += nthreads) {
        const int pp = e / A, a = e - pp * A;
        const float u0 = Ub[pp * us + a], u1 = Ub[pp * us + a + A];
        Ub[pp * us + a] = u0 * CS[a] - u1 * SN[a];
        Ub[pp * us + a + A] = u0 * SN[a] + u1 * CS[a];
      }
      __syncthreads();
      const float dec = aux[kAuxDecay];
      if (mma_wave) {
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          if (nb < p.NT) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              Hacc[nb][r] = fmaf(dec, Hacc[nb][r], Ub[(p0 + l16) * us + nb * 16 + 4 * lq + r]);
          }
        }
      }
      if (tid < A) run[tid] += aux[tid];
      __syncthreads();
    }
    for (int i = tid; i < p.PT * 16 * us; i += nthreads) Ub[i] = 0.f;  // restore the zero padding
  }
  float seg_decay = 1.f;  // thread 0: product of chunk decays (summary pass)

  // ---- register prefetch of one chunk's global operands -------------------
  // Addresses are a wave-uniform chunk base (scalar registers) plus a 32-bit
  // per-lane offset, so loads use the scalar-base + vector-offset form.
  const int xrow = P / VEC;   // x items per token
  const int brow = N / VEC;   // B / C items per virtual row
  const int tokx = p.H * P;   // x / z / out elements per token
  const int tokb = RG * N;    // B / C elements per token
  vec_t xr[KX], br[KB], cr[KB];
  float angr[KA];
  float s_dt = 0.f, s_adt = 0.f, s_trap = 0.f;

  auto prefetch = [&](int cs) {
    const int nv = min(Qt, t_end - cs);
    const float* xbase = p.x + (((size_t)b * p.L + cs) * p.H + h) * P;
    const float* bbase = p.b + ((size_t)b * p.L + cs) * tokb;
    const float* cbase = p.c + ((size_t)b * p.L + cs) * tokb;
    const float* abase = p.angle + ((size_t)b * p.L + cs) * A;
#pragma unroll
    for (int k = 0; k < KX; ++k) {
      const int idx = tid + k * nthreads;
      const int t = idx / xrow, pv = idx - t * xrow;
      vec_t v{};
      if (idx < Qt * xrow && t < nv) v = vload<VEC>(xbase + (uint32_t)(t * tokx + pv * VEC));
      xr[k] = v;
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int idx = tid + k * nthreads;
      const int u = idx / brow, j = idx - u * brow;
      const int t = u / R, r = u - t * R;
      vec_t v0{}, w0{};
      if (idx < Qt * R * brow && t < nv) {
        const uint32_t off = (uint32_t)(t * tokb + (r * p.G + g) * N + j * VEC);
        v0 = vload<VEC>(bbase + off);
        if (FULL) w0 = vload<VEC>(cbase + off);
      }
      br[k] = v0;
      cr[k] = w0;
    }
#pragma unroll
    for (int i = 0; i < KA; ++i) {
      const int a = 2 * (i * nwaves + wave) + (lane >> 5);
      const int t = lane & 31;
      angr[i] = (a < A && t < nv) ? abase[(uint32_t)(t * A + a)] : 0.f;
    }
    if (wave == 0) {
      const bool okl = lane <= Qt && cs + lane < p.L;
      const size_t sbase = ((size_t)b * p.L + cs) * p.H + h;
      const uint32_t so = (uint32_t)(lane * p.H);
      s_dt = okl ? p.dt[sbase + so] : 0.f;
      s_trap = okl ? p.trap[sbase + so] : 0.f;
      s_adt = lane < nv ? p.adt[sbase + so] : 0.f;
    }
  };

  prefetch(t_begin);
  __syncthreads();

  for (int c0 = t_begin; c0 < t_end; c0 += Qt) {
    const int nvalid = min(Qt, t_end - c0);

    // ---- P0: scalars (wave 0, lane = token); x, B, C rows into LDS; z loads --
    if (wave == 0) {
      const int t = lane;
      const float dt_n = next_lane_f(s_dt);
      const float tr_n = next_lane_f(s_trap);
      const bool ok = t < nvalid;
      const float dt_v = ok ? s_dt : 0.f;
      const float adt_v = ok ? s_adt : 0.f;
      const float gam = ok ? sigmoidf_acc(s_trap) * dt_v : 0.f;
      float scl = gam;
      if (ok && c0 + t + 1 < p.L) scl = gam + (1.f - sigmoidf_acc(tr_n)) * dt_n;
      const float cum = scan64_f(adt_v);
      const float cum_last = read_lane_f(cum, 63);  // padding lanes add zero
      if (t < Qt) {
        sc_cum[t] = cum;
        sc_ecum[t] = expf(cum);
        sc_gam[t] = gam;
        sc_scl[t] = scl;
        sc_w[t] = ok ? expf(cum_last - cum) * scl : 0.f;
        sc_dt[t] = dt_v;
      }
      if (lane == 0) {
        const float dec = expf(cum_last);
        run[64] = dec;
        seg_decay *= dec;
      }
    }
#pragma unroll
    for (int k = 0; k < KX; ++k) {
      const int idx = tid + k * nthreads;
      if (idx < Qt * xrow) {
        const int t = idx / xrow, pv = idx - t * xrow;
        if constexpr (MIMO) {
          for (int r = 0; r < R; ++r) {
            vec_t v = xr[k];
#pragma unroll
            for (int e = 0; e < VEC; ++e) set_comp(v, e, comp(v, e) * mxL[r * P + pv * VEC + e]);
            vstore<VEC>(Xl + ((t << rsl) + r) * xs + pv * VEC, v);
          }
        } else {
          vstore<VEC>(Xl + t * xs + pv * VEC, xr[k]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int idx = tid + k * nthreads;
      if (idx < Qt * R * brow) {
        const int u = idx / brow, j = idx - u * brow;
        const int t = u / R, r = u - t * R;
        const int v = (t << rsl) + r;
        const bool ok = t < nvalid;
        vec_t kv = br[k], qv = cr[k];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          set_comp(kv, e, ok ? comp(kv, e) + bbL[r * N + j * VEC + e] : 0.f);
          if (FULL) set_comp(qv, e, ok ? comp(qv, e) + cbL[r * N + j * VEC + e] : 0.f);
        }
        vstore<VEC>(Kl + v * ks + j * VEC, kv);
        if (FULL) vstore<VEC>(Ql + v * ks + j * VEC, qv);
      }
    }
    vec_t zr[KX];
    float zm[KZM][2];
    const size_t cbase_tok = (((size_t)b * p.L + c0) * p.H + h) * P;  // x / z / out at token c0
    const float* zbase = p.z + cbase_tok;
    if constexpr (FULL && !MIMO) {
#pragma unroll
      for (int k = 0; k < KX; ++k) {
        const int idx = tid + k * nthreads;
        const int t = idx / xrow, pv = idx - t * xrow;
        vec_t v{};
        if (p.has_z && idx < Qt * xrow && t < nvalid) v = vload<VEC>(zbase + (uint32_t)(t * tokx + pv * VEC));
        zr[k] = v;
      }
    }
    if constexpr (FULL && MIMO) {
#pragma unroll
      for (int i = 0; i < KZM; ++i) {
        const int t = wave + i * nwaves;
        const uint32_t ob = (uint32_t)(t * tokx);
        const bool ok = p.has_z && t < nvalid;
        zm[i][0] = (ok && lane < P) ? zbase[ob + lane] : 0.f;
        zm[i][1] = (ok && lane + 64 < P) ? zbase[ob + lane + 64] : 0.f;
      }
    }
    lds_barrier();

    // ---- P2: cumulative angle (32-lane scans), cos / sin, and the rotation of
    //      the pairs (a, a + A) of every rank's key and query row, in place -----
#pragma unroll
    for (int i = 0; i < KA; ++i) {
      const int am = 2 * (i * nwaves + wave);
      if (am >= A) break;  // wave-uniform
      const int a = am + (lane >> 5);
      const int t = lane & 31;
      const bool ok = a < A && t < nvalid;
      const float phi = scan32_f(ok ? sc_dt[t] * angr[i] : 0.f);
      if (ok) {
        const float th = run[a] + phi;
        float sn, co;
        sincos_acc(th, &sn, &co);
        for (int r = 0; r < R; ++r) {
          float* kr = Kl + ((t << rsl) + r) * ks;
          const float k0 = kr[a], k1 = kr[a + A];
          kr[a] = k0 * co - k1 * sn;
          kr[a + A] = k0 * sn + k1 * co;
          if (FULL) {
            float* qr = Ql + ((t << rsl) + r) * ks;
            const float q0 = qr[a], q1 = qr[a + A];
            qr[a] = q0 * co - q1 * sn;
            qr[a + A] = q0 * sn + q1 * co;
          }
        }
        if (t == nvalid - 1) run[a] = th;
      }
    }
    // The next chunk's loads go out now and land during this chunk's MFMA work.
    if (c0 + Qt < t_end) prefetch(c0 + Qt);
    lds_barrier();

    if constexpr (FULL) {
      // ---- P4: S = Q K^T on lower 16x16 tiles, masked ------------------------
      constexpr int NPAIRS = TB * (TB + 1) / 2;
      for (int pr = wave; pr < NPAIRS; pr += nwaves) {
        int tb = 0, sb = pr;
        while (sb > tb) { sb -= tb + 1; ++tb; }
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        const float* qa = Ql + (tb * 16 + l16) * ks + 4 * lq;
        const float* kb = Kl + (sb * 16 + l16) * ks + 4 * lq;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          if (nb < p.NT) {
            const floatx4 a4 = lds_read4(qa + nb * 16);
            const floatx4 b4 = lds_read4(kb + nb * 16);
            acc = mfma16(a4.x, b4.x, acc);
            acc = mfma16(a4.y, b4.y, acc);
            acc = mfma16(a4.z, b4.z, acc);
            acc = mfma16(a4.w, b4.w, acc);
          }
        }
        const int vs = sb * 16 + l16;
        const int ts_ = vs >> rsl;
        const float cum_s = sc_cum[ts_], scl_s = sc_scl[ts_];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int vt = tb * 16 + 4 * lq + r;
          const int tt = vt >> rsl;
          float m = 0.f;
          if (ts_ < tt) m = acc[r] * (exp_fast(sc_cum[tt] - cum_s) * scl_s);
          else if (ts_ == tt) m = acc[r] * sc_gam[tt];
          Ml[vt * ms + vs] = m;
        }
      }
      lds_barrier();
    }

    if (mma_wave) {
      if constexpr (FULL) {
        // ---- P5a: Y = M X + diag(exp(cum)) Q h'^T (this wave's 16 columns) ---
        for (int tb = 0; tb < TB; ++tb) {
          floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
          for (int sb = 0; sb <= tb; ++sb) {
            const floatx4 a4 = lds_read4(Ml + (tb * 16 + l16) * ms + sb * 16 + 4 * lq);
            const float* xc = Xl + (sb * 16 + 4 * lq) * xs + p0 + l16;
            acc = mfma16(a4.x, xc[0], acc);
            acc = mfma16(a4.y, xc[xs], acc);
            acc = mfma16(a4.z, xc[2 * xs], acc);
            acc = mfma16(a4.w, xc[3 * xs], acc);
          }
          const float ec = sc_ecum[(tb * 16 + l16) >> rsl];
          const float* qa = Ql + (tb * 16 + l16) * ks + 4 * lq;
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            if (nb < p.NT) {
              const floatx4 a4 = lds_read4(qa + nb * 16) * ec;
              acc = mfma16(a4.x, Hacc[nb].x, acc);
              acc = mfma16(a4.y, Hacc[nb].y, acc);
              acc = mfma16(a4.z, Hacc[nb].z, acc);
              acc = mfma16(a4.w, Hacc[nb].w, acc);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) Yl[(tb * 16 + 4 * lq + r) * ys + p0 + l16] = acc[r];
        }
      }
      // ---- P5b: state update h' = decay h' + K^T (w X) ------------------------
      const float dec = run[64];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) Hacc[nb] *= dec;
      for (int sb = 0; sb < TB; ++sb) {
        const int v0 = sb * 16 + 4 * lq;
        const float* xc = Xl + v0 * xs + p0 + l16;
        const float xw0 = xc[0] * sc_w[(v0 + 0) >> rsl];
        const float xw1 = xc[xs] * sc_w[(v0 + 1) >> rsl];
        const float xw2 = xc[2 * xs] * sc_w[(v0 + 2) >> rsl];
        const float xw3 = xc[3 * xs] * sc_w[(v0 + 3) >> rsl];
        const float* kc = Kl + v0 * ks + l16;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          if (nb < p.NT) {
            Hacc[nb] = mfma16(kc[nb * 16], xw0, Hacc[nb]);
            Hacc[nb] = mfma16(kc[ks + nb * 16], xw1, Hacc[nb]);
            Hacc[nb] = mfma16(kc[2 * ks + nb * 16], xw2, Hacc[nb]);
            Hacc[nb] = mfma16(kc[3 * ks + nb * 16], xw3, Hacc[nb]);
          }
        }
      }
    }
    lds_barrier();

    // ---- P6: epilogue ---------------------------------------------------------
    if constexpr (FULL && !MIMO) {
      // out = (y + D x) * silu(z), VEC-wide and coalesced along head_dim
      const float dh = p.has_d ? p.d[h] : 0.f;
#pragma unroll
      for (int k = 0; k < KX; ++k) {
        const int idx = tid + k * nthreads;
        const int t = idx / xrow, pv = idx - t * xrow;
        if (idx < Qt * xrow && t < nvalid) {
          vec_t y = vload<VEC>(Yl + t * ys + pv * VEC);
          const vec_t xv = vload<VEC>(Xl + t * xs + pv * VEC);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            float v = comp(y, e);
            if (p.has_d) v = fmaf(dh, comp(xv, e), v);
            if (p.has_z) v *= silu_fast(comp(zr[k], e));
            set_comp(y, e, v);
          }
          vstore<VEC>(p.out + cbase_tok + (uint32_t)(t * tokx + pv * VEC), y);
        }
      }
      lds_barrier();
    }
    if constexpr (FULL && MIMO) {
      // per rank: D skip, gate silu(z * mimo_z), optional RMS norm over P,
      // then the mimo_o-weighted sum over ranks; one wave per token
      const float dh = p.has_d ? p.d[h] : 0.f;
      const int pa = lane, pb = lane + 64;
#pragma unroll
      for (int i = 0; i < KZM; ++i) {
        const int t = wave + i * nwaves;
        if (t >= nvalid) break;  // wave-uniform
        float o0 = 0.f, o1 = 0.f;
        for (int r = 0; r < R; ++r) {
          const int v = (t << rsl) + r;
          float y0 = 0.f, y1 = 0.f;
          if (pa < P) {
            y0 = Yl[v * ys + pa];
            if (p.has_d) y0 = fmaf(dh, Xl[v * xs + pa], y0);
            if (p.has_z) y0 *= silu_fast(zm[i][0] * mzL[r * P + pa]);
          }
          if (pb < P) {
            y1 = Yl[v * ys + pb];
            if (p.has_d) y1 = fmaf(dh, Xl[v * xs + pb], y1);
            if (p.has_z) y1 *= silu_fast(zm[i][1] * mzL[r * P + pb]);
          }
          if (p.has_norm) {
            const float ss = read_lane_f(scan64_f(y0 * y0 + y1 * y1), 63);
            const float inv = 1.f / sqrtf(ss / (float)P + kNormEps);
            if (pa < P) y0 = y0 * inv * nwL[pa];
            if (pb < P) y1 = y1 * inv * nwL[pb];
          }
          if (pa < P) o0 = fmaf(moL[r * P + pa], y0, o0);
          if (pb < P) o1 = fmaf(moL[r * P + pb], y1, o1);
        }
        float* ob = p.out + cbase_tok + (uint32_t)(t * tokx);
        if (pa < P) ob[pa] = o0;
        if (pb < P) ob[pb] = o1;
      }
      lds_barrier();
    }
  }

  if constexpr (!FULL) {
    const size_t si = (size_t)bh * (p.nseg - 1) + seg;
    float* st = p.ws_state + si * (size_t)(p.PT * p.NT) * 256;
    if (mma_wave) {
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        if (nb < p.NT) *reinterpret_cast<floatx4*>(st + ((wave * p.NT + nb) * 64 + lane) * 4) = Hacc[nb];
    }
    float* aux = p.ws_aux + si * kAux;
    if (tid < A) aux[tid] = run[tid];
    if (tid == 0) aux[kAuxDecay] = seg_decay;
  }
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

int rank_stride(int R) {
  int RS = 1;
  while (RS < R) RS <<= 1;
  return RS;
}

ScanPlan make_plan(const ScanGeom& g) {
  ScanPlan pl{};
  pl.chunk = kQV;
  const int Qt = kQV / rank_stride((int)g.R);
  const int NT = ((int)g.N + 15) / 16, PT = ((int)g.P + 15) / 16;
  const long bhn = (long)g.B * g.H;
  // Split the sequence into as many segments as keep every workgroup resident
  // at once (two per CU on 256 CUs), so no CU runs a second round; each
  // segment keeps at least four chunks.
  const int target = env_int("M3_SCAN_TARGET_WG", 512);
  long nseg = 1;
  if (bhn < target) nseg = target / bhn;
  const long max_seg = ((long)g.L + 4L * Qt - 1) / (4L * Qt);
  if (nseg > max_seg) nseg = max_seg;
  const int forced = env_int("M3_SCAN_NSEG", 0);
  if (forced > 0) nseg = forced;
  if (nseg < 1) nseg = 1;
  long seg_len = ((long)g.L + nseg - 1) / nseg;
  seg_len = (seg_len + Qt - 1) / Qt * Qt;
  nseg = ((long)g.L + seg_len - 1) / seg_len;
  pl.nseg = (int)nseg;
  pl.seg_len = (int)seg_len;
  pl.ws_state_floats = nseg > 1 ? (size_t)bhn * (nseg - 1) * PT * NT * 256 : 0;
  pl.ws_aux_floats = nseg > 1 ? (size_t)bhn * (nseg - 1) * kAux : 0;
  return pl;
}

// LDS layout of one pass; the summary pass needs no Q, M or Y buffers.  Rows
// are padded by four floats so that rows 4 apart start 16 banks apart.
void layout(ScanKParams& kp, bool full, bool mimo) {
  const int QV = kQV;
  kp.ks = kp.NT * 16 + 4;
  kp.xs = kp.PT * 16 + 4;
  kp.ms = QV + 4;
  kp.ys = kp.PT * 16 + 4;
  int off = 0;
  kp.o_ql = off; off += full ? QV * kp.ks : 0;
  kp.o_kl = off; off += QV * kp.ks;
  kp.o_xl = off; off += QV * kp.xs;
  kp.o_ml = off; off += full ? QV * kp.ms : 0;
  kp.o_yl = off; off += full ? QV * kp.ys : 0;
  // the entry-state fold overlays [PT*16][NT*16+4] floats on the chunk buffers
  if (full && off < kp.PT * 16 * (kp.NT * 16 + 4)) off = kp.PT * 16 * (kp.NT * 16 + 4);
  kp.o_cs = off; off += 2 * 64;
  kp.o_bias = off; off += 2 * kp.R * kp.N;
  kp.o_mimo = off; off += mimo ? 3 * kp.R * kp.P + kp.P : 0;
  off = (off + 3) / 4 * 4;
  kp.o_sc = off; off += 6 * QV;
  kp.o_run = off; off += 68;
  kp.lds_floats = off;
}

template <int VEC, bool FULL, bool MIMO>
hipError_t launch_one(const ScanKParams& kp, unsigned grid, unsigned block, hipStream_t stream) {
  const size_t lds_bytes = (size_t)kp.lds_floats * sizeof(float);
  // Dynamic LDS above 64 KiB needs the opt-in attribute on some runtimes;
  // raise it when a larger layout first appears, and keep going if the
  // runtime does not know the attribute.
  static size_t attr_bytes = 64 * 1024;
  if (lds_bytes > attr_bytes) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_chunk_kernel<VEC, FULL, MIMO>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes) != hipSuccess)
      (void)hipGetLastError();
    attr_bytes = lds_bytes;
  }
  hipLaunchKernelGGL((scan_chunk_kernel<VEC, FULL, MIMO>), dim3(grid), dim3(block), lds_bytes, stream, kp);
  return hipGetLastError();
}

template <int VEC, bool MIMO>
hipError_t launch_passes(ScanKParams kp, const ScanPlan& plan, unsigned bhn, unsigned block,
                         hipStream_t stream) {
  if (plan.nseg > 1) {
    ScanKParams ka = kp;
    layout(ka, false, MIMO);
    hipError_t e = launch_one<VEC, false, MIMO>(ka, bhn * (unsigned)(plan.nseg - 1), block, stream);
    if (e != hipSuccess) return e;
  }
  layout(kp, true, MIMO);
  const ProfileEvents& pe = profile_events();
  if (pe.start) {
    hipError_t e = hipEventRecord(pe.start, stream);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_one<VEC, true, MIMO>(kp, bhn * (unsigned)plan.nseg, block, stream);
  if (e == hipSuccess && pe.stop) e = hipEventRecord(pe.stop, stream);
  return e;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0u; }

hipError_t launch_scan(const ScanGeom& g, const ScanOperands& o, const ScanPlan& plan,
                       void* workspace, hipStream_t stream) {
  ScanKParams kp{};
  kp.c = o.c; kp.b = o.b; kp.x = o.x; kp.z = o.z; kp.adt = o.adt; kp.dt = o.dt;
  kp.trap = o.trap; kp.angle = o.angle; kp.c_bias = o.c_bias; kp.b_bias = o.b_bias; kp.d = o.d;
  kp.mimo_x = o.mimo_x; kp.mimo_z = o.mimo_z; kp.mimo_o = o.mimo_o; kp.norm_weight = o.norm_weight;
  kp.out = o.out;
  kp.B = g.B; kp.L = g.L; kp.H = g.H; kp.G = g.G; kp.P = g.P; kp.N = g.N; kp.A = g.A; kp.R = g.R;
  kp.has_z = g.has_z; kp.has_d = g.has_d; kp.has_norm = g.has_norm;
  const bool mimo = o.mimo_x != nullptr;
  kp.NT = ((int)g.N + 15) / 16;
  kp.PT = ((int)g.P + 15) / 16;
  kp.RS = rank_stride((int)g.R);
  kp.rs_log2 = 0;
  while ((1 << kp.rs_log2) < kp.RS) ++kp.rs_log2;
  kp.Qt = kQV / kp.RS;
  kp.seg_len = plan.seg_len;
  kp.nseg = plan.nseg;
  float* ws = static_cast<float*>(workspace);
  kp.ws_state = ws;
  kp.ws_aux = ws ? ws + plan.ws_state_floats : nullptr;
  // 16-byte vector access needs every row width and row start on a 16-byte boundary.
  const bool vec4 = g.P % 4 == 0 && g.N % 4 == 0 && aligned16(o.x) && aligned16(o.z) && aligned16(o.b) && aligned16(o.c) &&
                    aligned16(o.out);
  // one wave per 16 head_dim columns, at least four, and enough that the
  // angle scan (two angles per wave and pass, four passes) covers A
  unsigned nwaves = kp.PT > 4 ? (unsigned)kp.PT : 4u;
  while (8u * nwaves < g.A) ++nwaves;
  const unsigned block = 64u * nwaves;
  const unsigned bhn = g.B * g.H;
  if (vec4)
    return mimo ? launch_passes<4, true>(kp, plan, bhn, block, stream)
                : launch_passes<4, false>(kp, plan, bhn, block, stream);
  return mimo ? launch_passes<1, true>(kp, plan, bhn, block, stream)
              : launch_passes<1, false>(kp, plan, bhn, block, stream);
}

}  // namespace

ProfileEvents& profile_events() {
  static thread_local ProfileEvents pe{nullptr, nullptr};
  return pe;
}

ScanPlan plan_siso(const ScanGeom& g) { return make_plan(g); }
ScanPlan plan_mimo(const ScanGeom& g) { return make_plan(g); }

hipError_t launch_siso_fwd(const ScanGeom& g, const ScanOperands& o, const ScanPlan& plan,
                           void* workspace, hipStream_t stream) {
  ScanOperands so = o;
  so.mimo_x = so.mimo_z = so.mimo_o = so.norm_weight = nullptr;
  return launch_scan(g, so, plan, workspace, stream);
}

hipError_t launch_mimo_fwd(const ScanGeom& g, const ScanOperands& o, const ScanPlan& plan,
                           void* workspace, hipStream_t stream) {
  return launch_scan(g, o, plan, workspace, stream);
}

}  // namespace m3
