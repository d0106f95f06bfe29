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
//   * A chunk holds QV "virtual rows" v = t * RS + r (token t, rank r < R,
//     RS = R rounded up to a power of two so that no token's rows straddle a
//     16-row MFMA tile; rows with r >= R stay zero).  SISO has R = RS = 1,
//     MIMO stacks its ranks inside the chunk.
//   * One workgroup runs one (batch, head, sequence segment); one wave per
//     16-wide slice of head_dim.  The state h'^T [N x P] lives in MFMA
//     accumulator registers for the whole segment: wave w keeps the 16x16
//     tiles (n-block, p-block w).
//   * Intra-chunk S = Q K^T, the decay/trapezoid mask, M X, the carried-state
//     read Q h'^T and the state update K^T (w X) all run on
//     v_mfma_f32_16x16x4_f32.
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

struct ScanKParams {
  const float *c, *b, *x, *z, *adt, *dt, *trap, *angle, *c_bias, *b_bias, *d;
  const float *mimo_x, *mimo_z, *mimo_o, *norm_weight;
  float* out;
  float* ws_state;  // [B*H][nseg-1][PT*NT tiles][64 lanes][4]
  float* ws_aux;    // [B*H][nseg-1][kAux]
  int B, L, H, G, P, N, A, R;
  int has_z, has_d, has_norm, mimo;
  int NT, PT;       // 16-wide blocks of N and P
  int RS, rs_log2;  // rank stride of the virtual rows (power of two >= R)
  int Qt;           // tokens per chunk (QV / RS)
  int seg_len, nseg;
  // LDS layout (float offsets) and row strides
  int o_ql, o_kt, o_xt, o_ml, o_yl, o_cs, o_sc, o_run, lds_floats;
  int ks, ts, ys;
};

template <int QV, bool FULL>
__global__ __launch_bounds__(512) void scan_chunk_kernel(ScanKParams p) {
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
  const int RS = p.RS, rsl = p.rs_log2;

  float* Ql = lds + p.o_ql;   // [QV][ks]   rotated C (+bias)
  float* Kt = lds + p.o_kt;   // [NT*16][ts] rotated B (+bias), transposed
  float* Xt = lds + p.o_xt;   // [PT*16][ts] per-rank x, transposed
  float* Ml = lds + p.o_ml;   // [QV][ts]   masked S
  float* Yl = lds + p.o_yl;   // [QV][ys]   raw y
  float* CS = lds + p.o_cs;   // [Qt][64] theta, then cos; [Qt][64] sin after it
  float* SN = CS + QV * 64;
  float* sc_cum = lds + p.o_sc;
  float* sc_ecum = sc_cum + QV;
  float* sc_gam = sc_ecum + QV;
  float* sc_scl = sc_gam + QV;
  float* sc_w = sc_scl + QV;
  float* sc_dt = sc_w + QV;
  float* run = lds + p.o_run;  // [0,64) running theta, [64] chunk decay

  for (int i = tid; i < p.lds_floats; i += nthreads) lds[i] = 0.f;
  __syncthreads();

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
    float* Ub = lds;  // [PT*16][NT*16 + 4], overlays the chunk buffers (unused yet)
    const int us = p.NT * 16 + 4;
    for (int i = 0; i < seg; ++i) {
      const size_t si = (size_t)bh * (p.nseg - 1) + i;
      const float* aux = p.ws_aux + si * kAux;
      const float* st = p.ws_state + si * (size_t)(p.PT * p.NT) * 256;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        if (nb < p.NT) {
          const floatx4 u = *reinterpret_cast<const floatx4*>(st + ((wave * p.NT + nb) * 64 + lane) * 4);
#pragma unroll
          for (int r = 0; r < 4; ++r) Ub[(p0 + l16) * us + nb * 16 + 4 * lq + r] = u[r];
        }
      }
      if (tid < p.A) {
        float sn, cs;
        sincosf(run[tid], &sn, &cs);
        CS[tid] = cs;
        SN[tid] = sn;
      }
      __syncthreads();
      for (int e = tid; e < p.PT * 16 * p.A; e += nthreads) {
        const int pp = e / p.A, a = e - pp * p.A;
        const float u0 = Ub[pp * us + a], u1 = Ub[pp * us + a + p.A];
        Ub[pp * us + a] = u0 * CS[a] - u1 * SN[a];
        Ub[pp * us + a + p.A] = u0 * SN[a] + u1 * CS[a];
      }
      __syncthreads();
      const float dec = aux[kAuxDecay];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        if (nb < p.NT) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Hacc[nb][r] = fmaf(dec, Hacc[nb][r], Ub[(p0 + l16) * us + nb * 16 + 4 * lq + r]);
        }
      }
      if (tid < p.A) run[tid] += aux[tid];
      __syncthreads();
    }
    for (int i = tid; i < p.PT * 16 * us; i += nthreads) Ub[i] = 0.f;  // restore the zero padding
  }
  float seg_decay = 1.f;  // thread 0: product of chunk decays (summary pass)
  __syncthreads();

  const int items_row = p.N - p.A;  // A rotated pairs + (N - 2A) plain coordinates per row

  for (int c0 = t_begin; c0 < t_end; c0 += Qt) {
    const int nvalid = min(Qt, t_end - c0);

    // ---- per-token scalars (wave 0; lane = token) -------------------------
    if (wave == 0) {
      const int t = lane;
      float adt_v = 0.f, dt_v = 0.f, gam = 0.f, scl = 0.f;
      if (t < nvalid) {
        const size_t idx = ((size_t)b * p.L + c0 + t) * p.H + h;
        dt_v = p.dt[idx];
        adt_v = p.adt[idx];
        gam = sigmoidf_acc(p.trap[idx]) * dt_v;
        scl = gam;
        if (c0 + t + 1 < p.L) {
          const size_t idn = idx + p.H;
          scl = gam + (1.f - sigmoidf_acc(p.trap[idn])) * p.dt[idn];
        }
      }
      float cum = adt_v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float v = __shfl_up(cum, off, 64);
        if (lane >= off) cum += v;
      }
      const float cum_last = __shfl(cum, 63, 64);  // padding lanes add zero
      if (t < Qt) {
        sc_cum[t] = cum;
        sc_ecum[t] = expf(cum);
        sc_gam[t] = gam;
        sc_scl[t] = scl;
        sc_w[t] = t < nvalid ? expf(cum_last - cum) * scl : 0.f;
        sc_dt[t] = dt_v;
      }
      if (lane == 0) {
        const float dec = expf(cum_last);
        run[64] = dec;
        seg_decay *= dec;
      }
    }
    __syncthreads();

    // ---- cumulative angle per token (thread a < A walks the chunk) ---------
    if (tid < p.A) {
      float th = run[tid];
      for (int t = 0; t < nvalid; ++t) {
        th = fmaf(sc_dt[t], p.angle[((size_t)b * p.L + c0 + t) * p.A + tid], th);
        CS[t * 64 + tid] = th;
      }
      run[tid] = th;
    }
    __syncthreads();
    for (int e = tid; e < nvalid * p.A; e += nthreads) {
      const int t = e / p.A, a = e - t * p.A;
      float s, co;
      sincosf(CS[t * 64 + a], &s, &co);
      CS[t * 64 + a] = co;
      SN[t * 64 + a] = s;
    }
    // ---- x rows (per rank) into Xt[p][v] ----------------------------------
    for (int e = tid; e < Qt * R * p.P; e += nthreads) {
      const int u = e / p.P, pp = e - u * p.P;
      const int t = u / R, r = u - t * R;
      const int v = (t << rsl) + r;
      float val = 0.f;
      if (t < nvalid) {
        val = p.x[(((size_t)b * p.L + c0 + t) * p.H + h) * p.P + pp];
        if (p.mimo) val *= p.mimo_x[((size_t)h * R + r) * p.P + pp];
      }
      Xt[pp * p.ts + v] = val;
    }
    __syncthreads();

    // ---- rotated keys / queries -------------------------------------------
    for (int e = tid; e < Qt * R * items_row; e += nthreads) {
      const int u = e / items_row, j = e - u * items_row;
      const int t = u / R, r = u - t * R;
      const int v = (t << rsl) + r;
      const bool ok = t < nvalid;
      const size_t row = (((size_t)b * p.L + c0 + t) * RG + r * p.G + g) * p.N;
      const size_t brow = ((size_t)h * R + r) * p.N;
      if (j < p.A) {
        const int a = j;
        float k0 = 0.f, k1 = 0.f, q0 = 0.f, q1 = 0.f;
        if (ok) {
          const float co = CS[t * 64 + a], s = SN[t * 64 + a];
          const float b0 = p.b[row + a] + p.b_bias[brow + a];
          const float b1 = p.b[row + a + p.A] + p.b_bias[brow + a + p.A];
          k0 = b0 * co - b1 * s;
          k1 = b0 * s + b1 * co;
          if (FULL) {
            const float e0 = p.c[row + a] + p.c_bias[brow + a];
            const float e1 = p.c[row + a + p.A] + p.c_bias[brow + a + p.A];
            q0 = e0 * co - e1 * s;
            q1 = e0 * s + e1 * co;
          }
        }
        Kt[a * p.ts + v] = k0;
        Kt[(a + p.A) * p.ts + v] = k1;
        if (FULL) {
          Ql[v * p.ks + a] = q0;
          Ql[v * p.ks + a + p.A] = q1;
        }
      } else {
        const int n = j + p.A;
        float k = 0.f, q = 0.f;
        if (ok) {
          k = p.b[row + n] + p.b_bias[brow + n];
          if (FULL) q = p.c[row + n] + p.c_bias[brow + n];
        }
        Kt[n * p.ts + v] = k;
        if (FULL) Ql[v * p.ks + n] = q;
      }
    }
    __syncthreads();

    constexpr int TB = QV / 16;
    if constexpr (FULL) {
      // ---- S = Q K^T on lower 16x16 tiles, masked -------------------------
      constexpr int NPAIRS = TB * (TB + 1) / 2;
      for (int pr = wave; pr < NPAIRS; pr += nwaves) {
        int tb = 0, sb = pr;
        while (sb > tb) { sb -= tb + 1; ++tb; }
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        const float* qa = Ql + (tb * 16 + l16) * p.ks + 4 * lq;
        const float* kb = Kt + (4 * lq) * p.ts + sb * 16 + l16;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          if (nb < p.NT) {
            const floatx4 a4 = lds_read4(qa + nb * 16);
            const float* kbn = kb + nb * 16 * p.ts;
            acc = mfma16(a4.x, kbn[0], acc);
            acc = mfma16(a4.y, kbn[p.ts], acc);
            acc = mfma16(a4.z, kbn[2 * p.ts], acc);
            acc = mfma16(a4.w, kbn[3 * p.ts], acc);
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
          if (ts_ < tt) m = acc[r] * (expf(sc_cum[tt] - cum_s) * scl_s);
          else if (ts_ == tt) m = acc[r] * sc_gam[tt];
          Ml[vt * p.ts + vs] = m;
        }
      }
      __syncthreads();

      // ---- Y = M X + diag(exp(cum)) Q h'^T  (this wave's 16 columns) -------
      for (int tb = 0; tb < TB; ++tb) {
        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
        for (int sb = 0; sb <= tb; ++sb) {
          const floatx4 a4 = lds_read4(Ml + (tb * 16 + l16) * p.ts + sb * 16 + 4 * lq);
          const floatx4 b4 = lds_read4(Xt + (p0 + l16) * p.ts + sb * 16 + 4 * lq);
          acc = mfma16(a4.x, b4.x, acc);
          acc = mfma16(a4.y, b4.y, acc);
          acc = mfma16(a4.z, b4.z, acc);
          acc = mfma16(a4.w, b4.w, acc);
        }
        const float ec = sc_ecum[(tb * 16 + l16) >> rsl];
        const float* qa = Ql + (tb * 16 + l16) * p.ks + 4 * lq;
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
        for (int r = 0; r < 4; ++r) Yl[(tb * 16 + 4 * lq + r) * p.ys + p0 + l16] = acc[r];
      }
    }

    // ---- state update h' = decay h' + K^T (w X) ---------------------------
    {
      const float dec = run[64];
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) Hacc[nb] *= dec;
      for (int sb = 0; sb < TB; ++sb) {
        floatx4 xw = lds_read4(Xt + (p0 + l16) * p.ts + sb * 16 + 4 * lq);
        const int v0 = sb * 16 + 4 * lq;
        xw.x *= sc_w[(v0 + 0) >> rsl];
        xw.y *= sc_w[(v0 + 1) >> rsl];
        xw.z *= sc_w[(v0 + 2) >> rsl];
        xw.w *= sc_w[(v0 + 3) >> rsl];
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
          if (nb < p.NT) {
            const floatx4 a4 = lds_read4(Kt + (nb * 16 + l16) * p.ts + sb * 16 + 4 * lq);
            Hacc[nb] = mfma16(a4.x, xw.x, Hacc[nb]);
            Hacc[nb] = mfma16(a4.y, xw.y, Hacc[nb]);
            Hacc[nb] = mfma16(a4.z, xw.z, Hacc[nb]);
            Hacc[nb] = mfma16(a4.w, xw.w, Hacc[nb]);
          }
        }
      }
    }
    __syncthreads();

    // ---- epilogue: D skip, gate, MIMO norm and rank mix; one wave per token
    if constexpr (FULL) {
      const float dh = p.has_d ? p.d[h] : 0.f;
      for (int t = wave; t < nvalid; t += nwaves) {
        const size_t ob = (((size_t)b * p.L + c0 + t) * p.H + h) * p.P;
        float o0 = 0.f, o1 = 0.f;
        const int pa = lane, pb = lane + 64;
        const float z0 = (p.has_z && pa < p.P) ? p.z[ob + pa] : 0.f;
        const float z1 = (p.has_z && pb < p.P) ? p.z[ob + pb] : 0.f;
        for (int r = 0; r < R; ++r) {
          const int v = (t << rsl) + r;
          float y0 = 0.f, y1 = 0.f;
          if (pa < p.P) {
            y0 = Yl[v * p.ys + pa];
            if (p.has_d) y0 = fmaf(dh, Xt[pa * p.ts + v], y0);
            if (p.has_z) y0 *= siluf_acc(p.mimo ? z0 * p.mimo_z[((size_t)h * R + r) * p.P + pa] : z0);
          }
          if (pb < p.P) {
            y1 = Yl[v * p.ys + pb];
            if (p.has_d) y1 = fmaf(dh, Xt[pb * p.ts + v], y1);
            if (p.has_z) y1 *= siluf_acc(p.mimo ? z1 * p.mimo_z[((size_t)h * R + r) * p.P + pb] : z1);
          }
          if (p.has_norm) {
            float ss = y0 * y0 + y1 * y1;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
            const float inv = 1.f / sqrtf(ss / (float)p.P + kNormEps);
            if (pa < p.P) y0 = y0 * inv * p.norm_weight[(size_t)h * p.P + pa];
            if (pb < p.P) y1 = y1 * inv * p.norm_weight[(size_t)h * p.P + pb];
          }
          if (p.mimo) {
            if (pa < p.P) o0 = fmaf(p.mimo_o[((size_t)h * R + r) * p.P + pa], y0, o0);
            if (pb < p.P) o1 = fmaf(p.mimo_o[((size_t)h * R + r) * p.P + pb], y1, o1);
          } else {
            o0 = y0;
            o1 = y1;
          }
        }
        if (pa < p.P) p.out[ob + pa] = o0;
        if (pb < p.P) p.out[ob + pb] = o1;
      }
      __syncthreads();
    }
  }

  if constexpr (!FULL) {
    const size_t si = (size_t)bh * (p.nseg - 1) + seg;
    float* st = p.ws_state + si * (size_t)(p.PT * p.NT) * 256;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      if (nb < p.NT) *reinterpret_cast<floatx4*>(st + ((wave * p.NT + nb) * 64 + lane) * 4) = Hacc[nb];
    float* aux = p.ws_aux + si * kAux;
    if (tid < p.A) aux[tid] = run[tid];
    if (tid == 0) aux[kAuxDecay] = seg_decay;
  }
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

constexpr int kQV = 32;

ScanPlan make_plan(const ScanGeom& g) {
  ScanPlan pl{};
  pl.chunk = kQV;
  const int R = (int)g.R;
  int RS = 1;
  while (RS < R) RS <<= 1;
  const int Qt = kQV / RS;
  const int NT = ((int)g.N + 15) / 16, PT = ((int)g.P + 15) / 16;
  const long bhn = (long)g.B * g.H;
  // Split the sequence into segments until there are enough workgroups to
  // cover the chip; each segment keeps at least a few chunks.
  int target = env_int("M3_SCAN_TARGET_WG", 256);
  long nseg = 1;
  if (bhn < target) nseg = (target + bhn - 1) / bhn;
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

template <int QV, bool FULL>
hipError_t launch_one(const ScanKParams& kp, unsigned grid, unsigned block, size_t lds_bytes,
                      hipStream_t stream) {
  // Dynamic LDS above 64 KiB needs the opt-in attribute on some runtimes;
  // set it once and keep going if the runtime does not know it.
  static bool attr_set = false;
  if (!attr_set && lds_bytes > 64 * 1024) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_chunk_kernel<QV, FULL>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes) != hipSuccess)
      (void)hipGetLastError();
    attr_set = true;
  }
  hipLaunchKernelGGL((scan_chunk_kernel<QV, FULL>), dim3(grid), dim3(block), lds_bytes, stream, kp);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanGeom& g, const ScanOperands& o, const ScanPlan& plan,
                       void* workspace, hipStream_t stream) {
  ScanKParams kp{};
  kp.c = o.c; kp.b = o.b; kp.x = o.x; kp.z = o.z; kp.adt = o.adt; kp.dt = o.dt;
  kp.trap = o.trap; kp.angle = o.angle; kp.c_bias = o.c_bias; kp.b_bias = o.b_bias; kp.d = o.d;
  kp.mimo_x = o.mimo_x; kp.mimo_z = o.mimo_z; kp.mimo_o = o.mimo_o; kp.norm_weight = o.norm_weight;
  kp.out = o.out;
  kp.B = g.B; kp.L = g.L; kp.H = g.H; kp.G = g.G; kp.P = g.P; kp.N = g.N; kp.A = g.A; kp.R = g.R;
  kp.has_z = g.has_z; kp.has_d = g.has_d; kp.has_norm = g.has_norm;
  kp.mimo = o.mimo_x != nullptr;
  kp.NT = ((int)g.N + 15) / 16;
  kp.PT = ((int)g.P + 15) / 16;
  kp.RS = 1;
  kp.rs_log2 = 0;
  while (kp.RS < (int)g.R) { kp.RS <<= 1; ++kp.rs_log2; }
  kp.Qt = kQV / kp.RS;
  kp.seg_len = plan.seg_len;
  kp.nseg = plan.nseg;
  float* ws = static_cast<float*>(workspace);
  kp.ws_state = ws;
  kp.ws_aux = ws ? ws + plan.ws_state_floats : nullptr;

  const int QV = kQV;
  kp.ks = kp.NT * 16 + 4;
  kp.ts = QV + 4;
  kp.ys = kp.PT * 16 + 4;
  int off = 0;
  kp.o_ql = off; off += QV * kp.ks;
  kp.o_kt = off; off += kp.NT * 16 * kp.ts;
  kp.o_xt = off; off += kp.PT * 16 * kp.ts;
  kp.o_ml = off; off += QV * kp.ts;
  kp.o_yl = off; off += QV * kp.ys;
  // the entry-state fold overlays [PT*16][NT*16+4] floats on the chunk buffers
  if (off < kp.PT * 16 * (kp.NT * 16 + 4)) off = kp.PT * 16 * (kp.NT * 16 + 4);
  kp.o_cs = off; off += 2 * QV * 64;
  kp.o_sc = off; off += 6 * QV;
  kp.o_run = off; off += 68;
  kp.lds_floats = off;
  const size_t lds_bytes = (size_t)off * sizeof(float);
  const unsigned block = 64u * (unsigned)kp.PT;
  const unsigned bhn = g.B * g.H;
  if (plan.nseg > 1) {
    hipError_t e = launch_one<kQV, false>(kp, bhn * (unsigned)(plan.nseg - 1), block, lds_bytes, stream);
    if (e != hipSuccess) return e;
  }
  const ProfileEvents& pe = profile_events();
  if (pe.start) {
    hipError_t e = hipEventRecord(pe.start, stream);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_one<kQV, true>(kp, bhn * (unsigned)plan.nseg, block, lds_bytes, stream);
  if (e == hipSuccess && pe.stop) e = hipEventRecord(pe.stop, stream);
  return e;
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
