// Mamba-3 SISO scan backward for gfx950: the adjoints of all eleven forward
// operands (mamba3_siso_backward of the oarust 0.8.6 page
// src/rs/ml/matrix/mamba3.rs; SsmBackward lists the gradients, one per
// operand in its layout).
//
// The forward, per (batch, head), in the running-state form
//     h'_t = a_t h'_{t-1} + s_t x_t K_t^T,   s_t = lam_t dt_t + (1-lam_{t+1}) dt_{t+1},
//     y_t  = a_t h'_{t-1} Q_t + lam_t dt_t (Q_t.K_t) x_t,
// has the state adjoint G_t (of h'_t) obeying G_{t-1} = a_t (G_t + gy_t Q_t^T)
// with gy_t = dout_t * silu(z_t).  Over a chunk of 32 tokens with entry
// state h'_e, exit adjoint G_x and chunk-local inclusive log-decay sums cum:
//     y   = diag(e^cum) Q h'_e^T + (M o Q K^T) X
//     dQ  = diag(e^cum) gy h'_e  + (M o gy X^T) K
//     dK  = diag(s e^(cumx-cum)) X G_x + (M o gy X^T)^T Q
//     GK  = diag(e^(cumx-cum)) K G_x^T + (V o Q K^T)^T gy      (row t: G_t K_t)
//     dx  = D gy + lam dt (Q.K) gy + s GK
// where M[t][s] = e^(cum_t-cum_s) s_s (s < t), lam_t dt_t (s = t), and
// V[r][t] = e^(cum_r-cum_t) (t < r).  The scalar adjoints follow from the
// per-token sums rho_t = gy_t.y_ssm_t, ds_t = x_t.GK_t, e_t = ds_t + (x_t.gy_t)(Q_t.K_t):
//     d gamma_t = e_t,  d c_t = ds_{t-1}  (c_t = (1-lam_t) dt_t),
//     d adt_t = Phi_t - gamma_t e_t,  Phi_t = sum_{r>=t} (rho_r - c_{r+1} ds_r - gamma_{r+1} e_{r+1}),
// the last being the reverse recurrence of <adjoint of h_t, h_t>.
//
// Launches: (1) cumulative angle per token and head; (2) per chunk, the
// forward summary sum_s e^(cumx-cum_s) s_s x_s K_s^T and the reverse summary
// sum_r e^(cum_r) gy_r Q_r^T on FP32 MFMA; (3) element-wise prefix over the
// chunks, turning them in place into entry states and exit adjoints;
// (4) per chunk, the products above on FP32 MFMA; (5) per token row, the
// rotation adjoints (angle derivative, un-rotation onto B/C + bias), the
// sum over the heads of a group and partial bias sums; (6) per head, the
// reverse sums over the sequence for adt, dt, trap and the angle; (7) the
// bias, D and angle reductions, all in a fixed order.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace m3 {
namespace {

constexpr int BQ = 32;     // tokens per chunk
constexpr int MS = BQ + 1; // row stride of the chunk-square matrices in LDS
constexpr int RB = 16;     // token rows per workgroup in the un-rotation pass

struct BwdK {
  const float *dout, *c, *b, *x, *z, *adt, *dt, *trap, *angle, *c_bias, *b_bias, *d;
  float *d_c, *d_b, *d_x, *d_z, *d_adt, *d_dt, *d_trap, *d_angle, *d_c_bias, *d_b_bias, *d_d;
  float* theta;     // [BH][L][A]   cumulative angle
  float* hs;        // [BH][nc][P][N] forward chunk summaries -> chunk-entry states h'
  float* gs;        // [BH][nc][P][N] reverse chunk summaries -> chunk-exit adjoints G
  float* decay;     // [BH][nc]     e^(sum of the chunk's adt)
  float* dtheta;    // [BH][L][A]   d theta -> the per-head angle adjoint
  float* dq_rot;    // [B][L][H][N] adjoint of the rotated query Q
  float* dk_rot;    // [B][L][H][N] adjoint of the rotated key K
  float* rho;       // [BH][L]
  float* dsv;       // [BH][L]
  float* ev;        // [BH][L]
  float* dd_part;   // [BH][nc]     per-chunk sum of x.gy
  float* bias_part; // [nrb][2][H][N] partial bias sums (0: b_bias, 1: c_bias)
  int B, L, H, G, P, N, A;
  int has_z, has_d;
  int nc, NT, PT, nrb;
};

__device__ __forceinline__ float dsilu_acc(float u) {
  const float s = sigmoidf_acc(u);
  return s * (1.f + u * (1.f - s));
}

// 16x16 block of A (16 x K) times B (K x 16), K a multiple of 4, operands in
// LDS with element (m, k) of A at a[m * am + k * ak] and (k, n) of B at
// bp[k * bk + n * bn].  Lane l reads A[l % 16][k0 + l / 16] and
// B[k0 + l / 16][l % 16], the operand layout of v_mfma_f32_16x16x4_f32.
__device__ __forceinline__ floatx4 mm_tile(const float* a, int am, int ak, const float* bp, int bk, int bn,
                                           int K, floatx4 acc, int lane) {
  const int r = lane & 15, q = lane >> 4;
  const float* ap = a + r * am + q * ak;
  const float* bq = bp + q * bk + r * bn;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 4) acc = mfma16(ap[k0 * ak], bq[k0 * bk], acc);
  return acc;
}

// Sum over the 16 lanes of each 16-lane row; the total lands in lane 15 of the row.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0x111>(v);
  v += dpp_f<0x112>(v);
  v += dpp_f<0x114>(v);
  v += dpp_f<0x118>(v);
  return v;
}

// Rotated, bias-added keys and queries of one chunk into LDS rows of stride
// ns (columns N .. ns-1 and rows past nv zero).  Column j < A pairs with
// j + A; A <= j < N - A stands for the plain column j + A.
__device__ void load_kq(const BwdK& p, int b, int h, int g, int t0, int nv, float* Kc, float* Qc, int ns,
                        int tid, int nthr) {
  const int N = p.N, A = p.A, NP = N - A, bh = b * p.H + h;
  const float* bb = p.b_bias + (size_t)h * N;
  const float* cb = p.c_bias + (size_t)h * N;
  for (int it = tid; it < BQ * NP; it += nthr) {
    const int t = it / NP, j = it - t * NP;
    const int n0 = j < A ? j : j + A;
    float k0 = 0.f, k1 = 0.f, q0 = 0.f, q1 = 0.f;
    if (t < nv) {
      const size_t row = (((size_t)b * p.L + t0 + t) * p.G + g) * N;
      if (j < A) {
        float sn, cs;
        sincos_acc(p.theta[((size_t)bh * p.L + t0 + t) * A + j], &sn, &cs);
        const float b0 = p.b[row + j] + bb[j], b1 = p.b[row + j + A] + bb[j + A];
        const float c0 = p.c[row + j] + cb[j], c1 = p.c[row + j + A] + cb[j + A];
        k0 = b0 * cs - b1 * sn;
        k1 = b0 * sn + b1 * cs;
        q0 = c0 * cs - c1 * sn;
        q1 = c0 * sn + c1 * cs;
      } else {
        k0 = p.b[row + n0] + bb[n0];
        q0 = p.c[row + n0] + cb[n0];
      }
    }
    Kc[t * ns + n0] = k0;
    Qc[t * ns + n0] = q0;
    if (j < A) {
      Kc[t * ns + j + A] = k1;
      Qc[t * ns + j + A] = q1;
    }
  }
  const int pad = ns - 1 - N;  // zero columns N .. 16 NT - 1
  for (int it = tid; it < BQ * pad; it += nthr) {
    const int t = it / pad, n = N + (it - t * pad);
    Kc[t * ns + n] = 0.f;
    Qc[t * ns + n] = 0.f;
  }
}

// (1) theta[bh][t][a] = sum_{s<=t} dt[b,s,h] angle[b,s,a]; one wave per (b, h).
__global__ __launch_bounds__(64) void bwd_theta_kernel(BwdK p) {
  const int bh = blockIdx.x, lane = threadIdx.x;
  const int b = bh / p.H, h = bh - b * p.H, A = p.A, L = p.L;
  if (lane >= A) return;
  float run = 0.f;
  const float* dtp = p.dt + (size_t)b * L * p.H + h;
  const float* ap = p.angle + (size_t)b * L * A + lane;
  float* out = p.theta + (size_t)bh * L * A + lane;
#pragma unroll 8
  for (int t = 0; t < L; ++t) {
    run = fmaf(dtp[(size_t)t * p.H], ap[(size_t)t * A], run);
    out[(size_t)t * A] = run;
  }
}

// Per-token scalars of a chunk into LDS (wave 0, lanes 0..31 own the tokens):
// cum (inclusive chunk-local sum of adt), s, gamma.  Tokens past the end
// get adt = s = gamma = 0, so cum stays flat there.
struct ChunkScalars {
  float* cum;
  float* scl;
  float* gam;
};

__device__ void chunk_scalars(const BwdK& p, int b, int h, int t0, int nv, const ChunkScalars& cs, int lane) {
  const int t = t0 + lane;
  float adt = 0.f, gam = 0.f, s = 0.f;
  if (lane < nv) {
    const size_t i = ((size_t)b * p.L + t) * p.H + h;
    adt = p.adt[i];
    const float dtv = p.dt[i];
    gam = sigmoidf_acc(p.trap[i]) * dtv;
    s = gam;
    if (t + 1 < p.L) {
      const size_t i1 = i + p.H;
      s += (1.f - sigmoidf_acc(p.trap[i1])) * p.dt[i1];
    }
  }
  const float cum = scan32_f(lane < 32 ? adt : 0.f);
  if (lane < BQ) {
    cs.cum[lane] = cum;
    cs.scl[lane] = s;
    cs.gam[lane] = gam;
  }
}

// (2) Per chunk: S = sum_s e^(cumx-cum_s) s_s x_s K_s^T and
// R = sum_r e^(cum_r) gy_r Q_r^T, both [P][N], and the chunk decay e^cumx.
__global__ __launch_bounds__(512) void bwd_summary_kernel(BwdK p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int NS = p.NT * 16 + 1, PS = p.PT * 16 + 1, PP = p.PT * 16, NN = p.NT * 16;
  float* Kc = lds;
  float* Qc = Kc + BQ * NS;
  float* Xw = Qc + BQ * NS;
  float* Gw = Xw + BQ * PS;
  float* cum = Gw + BQ * PS;
  float* scl = cum + BQ;
  float* gam = scl + BQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int bh = blockIdx.x / p.nc, c = blockIdx.x - bh * p.nc;
  const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
  const int t0 = c * BQ, nv = min(BQ, p.L - t0);
  if (wave == 0) chunk_scalars(p, b, h, t0, nv, ChunkScalars{cum, scl, gam}, lane);
  load_kq(p, b, h, g, t0, nv, Kc, Qc, NS, tid, blockDim.x);
  __syncthreads();
  const float cumx = cum[BQ - 1];
  for (int it = tid; it < BQ * PP; it += blockDim.x) {
    const int t = it / PP, pp = it - t * PP;
    float xw = 0.f, gw = 0.f;
    if (t < nv && pp < p.P) {
      const size_t gi = (((size_t)b * p.L + t0 + t) * p.H + h) * p.P + pp;
      float gy = p.dout[gi];
      if (p.has_z) gy *= siluf_acc(p.z[gi]);
      xw = expf(cumx - cum[t]) * scl[t] * p.x[gi];
      gw = expf(cum[t]) * gy;
    }
    Xw[t * PS + pp] = xw;
    Gw[t * PS + pp] = gw;
  }
  __syncthreads();
  if (tid == 0) p.decay[blockIdx.x] = expf(cumx);
  const int ntile = p.PT * p.NT;
  const size_t base = (size_t)blockIdx.x * p.P * p.N;
  const int r = lane & 15, q = lane >> 4;
  for (int job = wave; job < 2 * ntile; job += nw) {
    const bool rev = job >= ntile;
    const int jt = rev ? job - ntile : job;
    const int pt = jt / p.NT, nt = jt - pt * p.NT;
    // [p][n] = sum_t W[t][p] V[t][n]: A[m=p][k=t] = W[t][p], B[k=t][n] = V[t][n]
    const float* W = rev ? Gw : Xw;
    const float* V = rev ? Qc : Kc;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mm_tile(W + pt * 16, 1, PS, V + nt * 16, NS, 1, BQ, acc, lane);
    float* dst = (rev ? p.gs : p.hs) + base;
    const int n = nt * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pp = pt * 16 + 4 * q + i;
      if (pp < p.P && n < p.N) dst[(size_t)pp * p.N + n] = acc[i];
    }
  }
  (void)NN;
}

// (3) Element-wise over the chunks of one (b, h): hs[c] <- state before chunk
// c; gs[c] <- adjoint after chunk c.  In place.
__global__ __launch_bounds__(256) void bwd_prefix_kernel(BwdK p, int blocks_per_bh) {
  const int bh = blockIdx.x / blocks_per_bh;
  const int e = (blockIdx.x - bh * blocks_per_bh) * blockDim.x + threadIdx.x;
  const int PN = p.P * p.N, nc = p.nc;
  if (e >= PN) return;
  float* hs = p.hs + (size_t)bh * nc * PN + e;
  float* gs = p.gs + (size_t)bh * nc * PN + e;
  const float* dec = p.decay + (size_t)bh * nc;
  float run = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float v = hs[(size_t)c * PN];
    hs[(size_t)c * PN] = run;
    run = fmaf(dec[c], run, v);
  }
  run = 0.f;
  for (int c = nc - 1; c >= 0; --c) {
    const float v = gs[(size_t)c * PN];
    gs[(size_t)c * PN] = run;
    run = fmaf(dec[c], run, v);
  }
}

// (4) Per chunk: y, GK, dQ, dK on FP32 MFMA; writes d_z, d_x, the rotated
// query/key adjoints and the per-token sums rho, ds, e and x.gy.
__global__ __launch_bounds__(512) void bwd_chunk_kernel(BwdK p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int NS = p.NT * 16 + 1, PS = p.PT * 16 + 1, PP = p.PT * 16, NN = p.NT * 16;
  float* Kc = lds;
  float* Qc = Kc + BQ * NS;
  float* X = Qc + BQ * NS;
  float* GY = X + BQ * PS;
  float* HE = GY + BQ * PS;
  float* GX = HE + PP * NS;
  float* MQK = GX + PP * NS;
  float* VV = MQK + BQ * MS;
  float* MSG = VV + BQ * MS;
  float* cum = MSG + BQ * MS;
  float* scl = cum + BQ;
  float* gam = scl + BQ;
  float* qk = gam + BQ;
  float* xg = qk + BQ;
  float* rho_part = xg + BQ;                // [BQ][PT]
  float* ds_part = rho_part + BQ * p.PT;    // [BQ][PT]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int bh = blockIdx.x / p.nc, c = blockIdx.x - bh * p.nc;
  const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
  const int t0 = c * BQ, nv = min(BQ, p.L - t0);
  const int P = p.P, N = p.N, H = p.H;
  const float Dh = p.has_d ? p.d[h] : 0.f;

  if (wave == 0) chunk_scalars(p, b, h, t0, nv, ChunkScalars{cum, scl, gam}, lane);
  load_kq(p, b, h, g, t0, nv, Kc, Qc, NS, tid, blockDim.x);
  for (int it = tid; it < BQ * PP; it += blockDim.x) {
    const int t = it / PP, pp = it - t * PP;
    float xv = 0.f, gy = 0.f;
    if (t < nv && pp < P) {
      const size_t gi = (((size_t)b * p.L + t0 + t) * H + h) * P + pp;
      xv = p.x[gi];
      gy = p.dout[gi];
      if (p.has_z) gy *= siluf_acc(p.z[gi]);
    }
    X[t * PS + pp] = xv;
    GY[t * PS + pp] = gy;
  }
  {
    const size_t base = (size_t)blockIdx.x * P * N;
    for (int it = tid; it < PP * NN; it += blockDim.x) {
      const int pp = it / NN, n = it - pp * NN;
      float he = 0.f, gx = 0.f;
      if (pp < P && n < N) {
        he = p.hs[base + (size_t)pp * N + n];
        gx = p.gs[base + (size_t)pp * N + n];
      }
      HE[pp * NS + n] = he;
      GX[pp * NS + n] = gx;
    }
  }
  __syncthreads();
  const float cumx = cum[BQ - 1];
  const int r = lane & 15, q = lane >> 4;

  // chunk-square products, masked: waves 0-3 Q K^T, waves 4-7 gy X^T
  for (int job = wave; job < 8; job += nw) {
    const bool sgx = job >= 4;
    const int mt = (job & 3) >> 1, st = job & 1;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!sgx)
      acc = mm_tile(Qc + mt * 16 * NS, NS, 1, Kc + st * 16 * NS, 1, NS, NN, acc, lane);
    else
      acc = mm_tile(GY + mt * 16 * PS, PS, 1, X + st * 16 * PS, 1, PS, PP, acc, lane);
    const int s = st * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = mt * 16 + 4 * q + i;
      const float v = acc[i];
      const float dec = s < t ? expf(cum[t] - cum[s]) : 0.f;
      const float m = s < t ? dec * scl[s] : (s == t ? gam[t] : 0.f);
      if (!sgx) {
        MQK[t * MS + s] = m * v;
        VV[t * MS + s] = dec * v;
        if (s == t) qk[t] = v;
      } else {
        MSG[t * MS + s] = m * v;
        if (s == t) xg[t] = v;
      }
    }
  }
  __syncthreads();

  const int nY = 2 * p.PT, nQ = 2 * p.NT;
  const int njobs = 2 * nY + 2 * nQ;
  for (int job = wave; job < njobs; job += nw) {
    floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
    if (job < 2 * nY) {
      const bool isgk = job >= nY;
      const int jj = isgk ? job - nY : job;
      const int mt = jj / p.PT, pt = jj - mt * p.PT;
      if (!isgk) {
        a1 = mm_tile(Qc + mt * 16 * NS, NS, 1, HE + pt * 16 * NS, 1, NS, NN, a1, lane);
        a2 = mm_tile(MQK + mt * 16 * MS, MS, 1, X + pt * 16, PS, 1, BQ, a2, lane);
      } else {
        a1 = mm_tile(Kc + mt * 16 * NS, NS, 1, GX + pt * 16 * NS, 1, NS, NN, a1, lane);
        a2 = mm_tile(VV + mt * 16, 1, MS, GY + pt * 16, PS, 1, BQ, a2, lane);
      }
      const int pp = pt * 16 + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + 4 * q + i;
        const bool ok = t < nv && pp < P;
        const size_t gi = (((size_t)b * p.L + t0 + t) * H + h) * P + pp;
        const float xv = X[t * PS + pp], gy = GY[t * PS + pp];
        float part;
        if (!isgk) {
          const float y = fmaf(expf(cum[t]), a1[i], a2[i]);
          part = gy * y;
          if (ok) {
            float dz = 0.f;
            if (p.has_z) {
              const float zv = p.z[gi];
              dz = p.dout[gi] * fmaf(Dh, xv, y) * dsilu_acc(zv);
            }
            p.d_z[gi] = dz;
          }
        } else {
          const float gk = fmaf(expf(cumx - cum[t]), a1[i], a2[i]);
          part = xv * gk;
          if (ok) p.d_x[gi] = fmaf(Dh + gam[t] * qk[t], gy, scl[t] * gk);
        }
        part = row16_sum(ok ? part : 0.f);
        if (r == 15) (isgk ? ds_part : rho_part)[t * p.PT + pt] = part;
      }
    } else {
      const bool isdk = job >= 2 * nY + nQ;
      const int jj = job - 2 * nY - (isdk ? nQ : 0);
      const int mt = jj / p.NT, nt = jj - mt * p.NT;
      if (!isdk) {
        a1 = mm_tile(GY + mt * 16 * PS, PS, 1, HE + nt * 16, NS, 1, PP, a1, lane);
        a2 = mm_tile(MSG + mt * 16 * MS, MS, 1, Kc + nt * 16, NS, 1, BQ, a2, lane);
      } else {
        a1 = mm_tile(X + mt * 16 * PS, PS, 1, GX + nt * 16, NS, 1, PP, a1, lane);
        a2 = mm_tile(MSG + mt * 16, 1, MS, Qc + nt * 16, NS, 1, BQ, a2, lane);
      }
      const int n = nt * 16 + r;
      float* dst = isdk ? p.dk_rot : p.dq_rot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + 4 * q + i;
        const float w = isdk ? scl[t] * expf(cumx - cum[t]) : expf(cum[t]);
        if (t < nv && n < N) dst[(((size_t)b * p.L + t0 + t) * H + h) * N + n] = fmaf(w, a1[i], a2[i]);
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    float xgv = 0.f;
    if (lane < nv) {
      float rh = 0.f, ds = 0.f;
      for (int pt = 0; pt < p.PT; ++pt) {
        rh += rho_part[lane * p.PT + pt];
        ds += ds_part[lane * p.PT + pt];
      }
      xgv = xg[lane];
      const size_t i = (size_t)bh * p.L + t0 + lane;
      p.rho[i] = rh;
      p.dsv[i] = ds;
      p.ev[i] = fmaf(xgv, qk[lane], ds);
    }
    const float tot = scan32_f(lane < 32 ? xgv : 0.f);
    if (lane == 31) p.dd_part[blockIdx.x] = tot;
  }
}

// (5) Per block of RB token rows (b, t) and group g: angle derivative per
// head, un-rotation of dK / dQ onto B + b_bias / C + c_bias, the sum over
// the group's heads into d_b / d_c, and partial bias sums.  Thread (hs, j)
// owns column pair j of heads hs, hs + nhs, ... for every row of the block.
__global__ __launch_bounds__(256) void bwd_unrotate_kernel(BwdK p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int N = p.N, A = p.A, NP = N - A, H = p.H, G = p.G, HG = H / G;
  const int g = blockIdx.y, blk = blockIdx.x;
  const int tid = threadIdx.x;
  const int nhs = max(1, (int)blockDim.x / NP);
  const int hs = tid / NP, j = tid - hs * NP;
  const bool active = hs < nhs && hs < HG;
  const int n0 = j < A ? j : j + A;
  float* bacc = lds;                 // [2][HG][N] bias sums of this block
  float* gsum = bacc + 2 * HG * N;   // [nhs][4][NP] group partials per head subset
  for (int i = tid; i < 2 * HG * N; i += blockDim.x) bacc[i] = 0.f;
  __syncthreads();
  const int rows = p.B * p.L;
  for (int rr = 0; rr < RB; ++rr) {
    const int row = blk * RB + rr;
    if (row >= rows) break;
    const int b = row / p.L, t = row - b * p.L;
    float gb0 = 0.f, gb1 = 0.f, gc0 = 0.f, gc1 = 0.f;
    if (active) {
      const size_t brow = ((size_t)row * G + g) * N;
      for (int hh = hs; hh < HG; hh += nhs) {
        const int h = g * HG + hh;
        const size_t di = ((size_t)row * H + h) * N;
        const float dk0 = p.dk_rot[di + n0], dq0 = p.dq_rot[di + n0];
        const float* bb = p.b_bias + (size_t)h * N;
        const float* cb = p.c_bias + (size_t)h * N;
        float ub0, ub1 = 0.f, uc0, uc1 = 0.f;
        if (j < A) {
          const float dk1 = p.dk_rot[di + j + A], dq1 = p.dq_rot[di + j + A];
          const size_t ti = (((size_t)b * H + h) * p.L + t) * A + j;
          float sn, cs;
          sincos_acc(p.theta[ti], &sn, &cs);
          const float b0 = p.b[brow + j] + bb[j], b1 = p.b[brow + j + A] + bb[j + A];
          const float c0 = p.c[brow + j] + cb[j], c1 = p.c[brow + j + A] + cb[j + A];
          const float K0 = b0 * cs - b1 * sn, K1 = b0 * sn + b1 * cs;
          const float Q0 = c0 * cs - c1 * sn, Q1 = c0 * sn + c1 * cs;
          p.dtheta[ti] = dk1 * K0 - dk0 * K1 + dq1 * Q0 - dq0 * Q1;
          ub0 = dk0 * cs + dk1 * sn;
          ub1 = dk1 * cs - dk0 * sn;
          uc0 = dq0 * cs + dq1 * sn;
          uc1 = dq1 * cs - dq0 * sn;
        } else {
          ub0 = dk0;
          uc0 = dq0;
        }
        gb0 += ub0;
        gb1 += ub1;
        gc0 += uc0;
        gc1 += uc1;
        bacc[hh * N + n0] += ub0;
        bacc[(HG + hh) * N + n0] += uc0;
        if (j < A) {
          bacc[hh * N + j + A] += ub1;
          bacc[(HG + hh) * N + j + A] += uc1;
        }
      }
      float* gp = gsum + (size_t)hs * 4 * NP;
      gp[j] = gb0;
      gp[NP + j] = gb1;
      gp[2 * NP + j] = gc0;
      gp[3 * NP + j] = gc1;
    }
    __syncthreads();
    if (tid < NP) {
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
      for (int k = 0; k < min(nhs, HG); ++k) {
        const float* gp = gsum + (size_t)k * 4 * NP;
        s0 += gp[tid];
        s1 += gp[NP + tid];
        s2 += gp[2 * NP + tid];
        s3 += gp[3 * NP + tid];
      }
      const int m0 = tid < A ? tid : tid + A;
      const size_t o = ((size_t)row * G + g) * N;
      p.d_b[o + m0] = s0;
      p.d_c[o + m0] = s2;
      if (tid < A) {
        p.d_b[o + tid + A] = s1;
        p.d_c[o + tid + A] = s3;
      }
    }
    __syncthreads();
  }
  for (int i = tid; i < 2 * HG * N; i += blockDim.x) {
    const int which = i / (HG * N), rem = i - which * HG * N;
    const int hh = rem / N, n = rem - hh * N;
    p.bias_part[(((size_t)blk * 2 + which) * H + g * HG + hh) * N + n] = bacc[i];
  }
}

// Inclusive suffix sum over the 64 lanes of a wave.
__device__ __forceinline__ float suffix64(float v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_down(v, off, 64);
    if (lane + off < 64) v += o;
  }
  return v;
}

// (6) Per (b, h), tokens in reverse tiles of 64: Phi, d adt, d dt, d trap,
// and the per-head angle adjoint dt_t * sum_{r>=t} d theta_r (in place).
__global__ __launch_bounds__(256) void bwd_finalize_kernel(BwdK p) {
  __shared__ float tile[64 * 65];
  __shared__ float carry[64];
  __shared__ float ddt_part[4][64];
  const int bh = blockIdx.x, b = bh / p.H, h = bh - b * p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = p.L, A = p.A, H = p.H;
  if (tid < 64) carry[tid] = 0.f;
  float phi_carry = 0.f;
  __syncthreads();
  for (int tlo = ((L - 1) / 64) * 64; tlo >= 0; tlo -= 64) {
    const int t = tlo + lane;
    const int nt = min(64, L - tlo);
    // the tile of d theta [64][A] into LDS
    for (int i = tid; i < 64 * A; i += blockDim.x) {
      const int tt = i / A, a = i - tt * A;
      tile[tt * 65 + a] = tt < nt ? p.dtheta[((size_t)bh * L + tlo + tt) * A + a] : 0.f;
    }
    __syncthreads();
    const bool ok = lane < nt;
    const size_t si = ((size_t)b * L + t) * H + h;
    const float dtv = ok ? p.dt[si] : 0.f;
    float part = 0.f;
    for (int a = wave; a < A; a += 4) {
      float v = suffix64(tile[lane * 65 + a], lane) + carry[a];
      if (ok) {
        p.dtheta[((size_t)bh * L + t) * A + a] = dtv * v;
        part = fmaf(v, p.angle[((size_t)b * L + t) * A + a], part);
      }
      // column a belongs to this wave alone; its LDS read above precedes this write
      const float tot = __shfl(v, 0, 64);
      if (lane == 0) carry[a] = tot;
    }
    ddt_part[wave][lane] = part;
    __syncthreads();
    if (wave == 0) {
      float psi = 0.f, lam = 0.f, e = 0.f, dc = 0.f, gamv = 0.f;
      if (ok) {
        const size_t ri = (size_t)bh * L + t;
        lam = sigmoidf_acc(p.trap[si]);
        gamv = lam * dtv;
        e = p.ev[ri];
        const float ds = p.dsv[ri];
        psi = p.rho[ri];
        if (t + 1 < L) {
          const size_t s1 = si + H;
          const float lam1 = sigmoidf_acc(p.trap[s1]), dt1 = p.dt[s1];
          psi -= (1.f - lam1) * dt1 * ds + lam1 * dt1 * p.ev[ri + 1];
        }
        if (t >= 1) dc = p.dsv[ri - 1];
      }
      const float phi = suffix64(psi, lane) + phi_carry;
      phi_carry = __shfl(phi, 0, 64);
      if (ok) {
        const float rot = ddt_part[0][lane] + ddt_part[1][lane] + ddt_part[2][lane] + ddt_part[3][lane];
        p.d_adt[si] = fmaf(-gamv, e, phi);
        p.d_dt[si] = fmaf(lam, e, fmaf(1.f - lam, dc, rot));
        p.d_trap[si] = lam * (1.f - lam) * dtv * (e - dc);
      }
    }
    __syncthreads();
  }
}

// (7a) d_c_bias, d_b_bias from the block partials; d_d from the chunk partials.
__global__ __launch_bounds__(256) void bwd_bias_kernel(BwdK p) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int HN = p.H * p.N;
  if (i < 2 * HN) {
    const int which = i / HN, rem = i - which * HN;
    float s = 0.f;
    for (int k = 0; k < p.nrb; ++k) s += p.bias_part[((size_t)k * 2 + which) * HN + rem];
    (which == 0 ? p.d_b_bias : p.d_c_bias)[rem] = s;
  } else if (i < 2 * HN + p.H) {
    const int h = i - 2 * HN;
    float s = 0.f;
    if (p.has_d)
      for (int bb = 0; bb < p.B; ++bb)
        for (int c = 0; c < p.nc; ++c) s += p.dd_part[((size_t)bb * p.H + h) * p.nc + c];
    p.d_d[h] = s;
  }
}

// (7b) d_angle[b][t][a] = sum_h (per-head angle adjoint).
__global__ __launch_bounds__(256) void bwd_angle_kernel(BwdK p) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)p.B * p.L * p.A;
  if (i >= total) return;
  const int a = (int)(i % p.A);
  const size_t bt = i / p.A;
  const int t = (int)(bt % p.L), b = (int)(bt / p.L);
  float s = 0.f;
  for (int h = 0; h < p.H; ++h) s += p.dtheta[(((size_t)b * p.H + h) * p.L + t) * p.A + a];
  p.d_angle[i] = s;
}

struct BwdLayout {
  size_t theta, hs, gs, decay, dtheta, dq, dk, rho, dsv, ev, ddp, bias, total;
  int nc, nrb;
};

BwdLayout bwd_layout(const ScanGeom& g) {
  BwdLayout w{};
  const size_t BH = (size_t)g.B * g.H;
  w.nc = (int)((g.L + BQ - 1) / BQ);
  w.nrb = (int)(((size_t)g.B * g.L + RB - 1) / RB);
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += (n + 63) / 64 * 64;  // 256-byte aligned pieces
    return o;
  };
  w.theta = take(BH * g.L * g.A);
  w.hs = take(BH * w.nc * g.P * g.N);
  w.gs = take(BH * w.nc * g.P * g.N);
  w.decay = take(BH * w.nc);
  w.dtheta = take(BH * g.L * g.A);
  w.dq = take((size_t)g.B * g.L * g.H * g.N);
  w.dk = take((size_t)g.B * g.L * g.H * g.N);
  w.rho = take(BH * g.L);
  w.dsv = take(BH * g.L);
  w.ev = take(BH * g.L);
  w.ddp = take(BH * w.nc);
  w.bias = take((size_t)w.nrb * 2 * g.H * g.N);
  w.total = off;
  return w;
}

size_t chunk_lds_bytes(int PT, int NT) {
  const int NS = NT * 16 + 1, PS = PT * 16 + 1, PP = PT * 16;
  return (size_t)(2 * BQ * NS + 2 * BQ * PS + 2 * PP * NS + 3 * BQ * MS + 5 * BQ + 2 * BQ * PT) * sizeof(float);
}

size_t summary_lds_bytes(int PT, int NT) {
  const int NS = NT * 16 + 1, PS = PT * 16 + 1;
  return (size_t)(2 * BQ * NS + 2 * BQ * PS + 3 * BQ) * sizeof(float);
}

void raise_lds(const void* fn, size_t bytes) {
  if (bytes > 64 * 1024 &&
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
    (void)hipGetLastError();
}

}  // namespace

size_t siso_bwd_workspace_floats(const ScanGeom& g) { return bwd_layout(g).total; }

bool siso_bwd_fits(const ScanGeom& g) {
  const int PT = (int)((g.P + 15) / 16), NT = (int)((g.N + 15) / 16);
  const int HG = (int)(g.H / g.G);
  const int nhs = (int)std::max(1u, 256u / (g.N - g.A));
  const size_t unrot = (size_t)(2 * HG * g.N + std::min(nhs, HG) * 4 * (g.N - g.A)) * sizeof(float);
  return chunk_lds_bytes(PT, NT) <= 160 * 1024 && unrot <= 160 * 1024;
}

hipError_t launch_siso_bwd(const ScanGeom& g, const ScanOperands& o, const BwdOperands& go, void* workspace,
                           hipStream_t stream) {
  const BwdLayout w = bwd_layout(g);
  float* ws = static_cast<float*>(workspace);
  BwdK k{};
  k.dout = go.dout;
  k.c = o.c; k.b = o.b; k.x = o.x; k.z = o.z; k.adt = o.adt; k.dt = o.dt; k.trap = o.trap;
  k.angle = o.angle; k.c_bias = o.c_bias; k.b_bias = o.b_bias; k.d = o.d;
  k.d_c = go.d_c; k.d_b = go.d_b; k.d_x = go.d_x; k.d_z = go.d_z; k.d_adt = go.d_adt; k.d_dt = go.d_dt;
  k.d_trap = go.d_trap; k.d_angle = go.d_angle; k.d_c_bias = go.d_c_bias; k.d_b_bias = go.d_b_bias;
  k.d_d = go.d_d;
  k.theta = ws + w.theta; k.hs = ws + w.hs; k.gs = ws + w.gs; k.decay = ws + w.decay;
  k.dtheta = ws + w.dtheta; k.dq_rot = ws + w.dq; k.dk_rot = ws + w.dk;
  k.rho = ws + w.rho; k.dsv = ws + w.dsv; k.ev = ws + w.ev; k.dd_part = ws + w.ddp;
  k.bias_part = ws + w.bias;
  k.B = (int)g.B; k.L = (int)g.L; k.H = (int)g.H; k.G = (int)g.G; k.P = (int)g.P; k.N = (int)g.N;
  k.A = (int)g.A; k.has_z = (int)g.has_z; k.has_d = (int)g.has_d;
  k.nc = w.nc; k.NT = (int)((g.N + 15) / 16); k.PT = (int)((g.P + 15) / 16); k.nrb = w.nrb;
  const unsigned BH = g.B * g.H;
  hipError_t e;
  if (g.A > 0) {
    hipLaunchKernelGGL(bwd_theta_kernel, dim3(BH), dim3(64), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const size_t sl = summary_lds_bytes(k.PT, k.NT);
  raise_lds(reinterpret_cast<const void*>(&bwd_summary_kernel), sl);
  hipLaunchKernelGGL(bwd_summary_kernel, dim3(BH * w.nc), dim3(512), sl, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned pnb = (g.P * g.N + 255) / 256;
  hipLaunchKernelGGL(bwd_prefix_kernel, dim3(pnb * BH), dim3(256), 0, stream, k, (int)pnb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t cl = chunk_lds_bytes(k.PT, k.NT);
  raise_lds(reinterpret_cast<const void*>(&bwd_chunk_kernel), cl);
  hipLaunchKernelGGL(bwd_chunk_kernel, dim3(BH * w.nc), dim3(512), cl, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int NP = (int)(g.N - g.A), HG = (int)(g.H / g.G);
  const int nhs = std::max(1, 256 / NP);
  const size_t ul = (size_t)(2 * HG * g.N + std::min(nhs, HG) * 4 * NP) * sizeof(float);
  raise_lds(reinterpret_cast<const void*>(&bwd_unrotate_kernel), ul);
  hipLaunchKernelGGL(bwd_unrotate_kernel, dim3(w.nrb, g.G), dim3(256), ul, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_finalize_kernel, dim3(BH), dim3(256), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned nb = (2u * g.H * g.N + g.H + 255u) / 256u;
  hipLaunchKernelGGL(bwd_bias_kernel, dim3(nb), dim3(256), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (g.A > 0) {
    const size_t tot = (size_t)g.B * g.L * g.A;
    hipLaunchKernelGGL(bwd_angle_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace m3
