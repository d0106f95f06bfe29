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
//     d adt_t = sum_{r>=t} (rho_r - c_{r+1} ds_r - gamma_r e_r),
// the last from the reverse recurrence of <adjoint of h_t, h_t>, which
// telescopes into a suffix sum of per-token terms.
//
// Launches: (1) chunk-local cumulative angles and (2) a scan of the tile
// totals; (3) per chunk, the forward summary sum_s e^(cumx-cum_s) s_s x_s K_s^T
// and the reverse summary sum_r e^(cum_r) gy_r Q_r^T on FP32 MFMA;
// (4) element-wise prefix over the chunks, turning them in place into entry
// states and exit adjoints; (5) per chunk, the products above on FP32 MFMA,
// the rotation adjoints (angle derivative, un-rotation onto B + b_bias and
// C + c_bias per head) and chunk-local suffix sums; (6) a scan of the chunk
// totals; (7) per chunk, d adt, d dt, d trap and the per-head angle adjoint;
// (8) per token row, the sum over a group's heads and partial bias sums;
// (9) the bias, D and angle reductions.  Every reduction has a fixed order,
// so results repeat bit for bit.  Each kernel issues its global loads
// together, so a workgroup waits on about one memory round trip.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace m3 {
namespace {

constexpr int BQ = 32;      // tokens per chunk
constexpr int MS = BQ + 1;  // row stride of the chunk-square matrices in LDS
constexpr int RB = 16;      // token rows per workgroup in the group reduction
constexpr int TT = 64;      // tokens per tile of the cumulative-angle scan
constexpr int KQ_ITEMS = 8; // (token, column pair) items per thread: 32 * 128 / 512
constexpr int KQ_ROUND = 4; // of which this many have their loads in flight together
constexpr int XG_ITEMS = 8; // (token, head_dim) items per thread: 32 * 128 / 512

struct BwdK {
  const float *dout, *c, *b, *x, *z, *adt, *dt, *trap, *angle, *c_bias, *b_bias, *d;
  float *d_c, *d_b, *d_x, *d_z, *d_adt, *d_dt, *d_trap, *d_angle, *d_c_bias, *d_b_bias, *d_d;
  float* theta;     // [BH][L][A]     cumulative angle within its 64-token tile
  float* tpre;      // [BH][nT][A]    sum of the angle increments of the earlier tiles
  float* hs;        // [BH][nc][P][N] forward chunk summaries -> chunk-entry states h'
  float* gs;        // [BH][nc][P][N] reverse chunk summaries -> chunk-exit adjoints G
  float* decay;     // [BH][nc]       e^(sum of the chunk's adt)
  float* dtheta;    // [BH][L][A]     chunk-local suffix of d theta -> per-head angle adjoint
  float* db_head;   // [B][L][H][N]   per-head adjoint of B + b_bias
  float* dc_head;   // [B][L][H][N]   per-head adjoint of C + c_bias
  float* dsv;       // [BH][L]        ds_t = x_t . G_t K_t
  float* ev;        // [BH][L]        e_t = ds_t + (x_t . gy_t)(Q_t . K_t)
  float* phi_tot;   // [BH][nc]       chunk sums of the d adt terms -> sums over later chunks
  float* th_tot;    // [BH][nc][A]    chunk sums of d theta -> sums over later chunks
  float* dd_part;   // [BH][nc]       per-chunk sum of x . gy
  float* bias_part; // [nrb][2][H][R N] partial bias sums (0: b_bias, 1: c_bias)
  // MIMO: per-rank weights and their gradients; the upstream gradient of each
  // rank's state read-out gy [BH][nc * BQ][P] (rows v = token * RS + rank);
  // per-chunk partial sums of the weight gradients
  const float *mimo_x, *mimo_z, *mimo_o, *norm_weight;
  float *d_mimo_x, *d_mimo_z, *d_mimo_o, *d_norm_weight;
  float* gyr;
  float* rho;       // [BH][L] gy . (state read-out), summed over ranks
  float *mx_part, *mz_part, *mo_part, *nw_part;  // [BH nc][R P] (nw: [BH nc][P])
  int B, L, H, G, P, N, A;
  int has_z, has_d, has_norm;
  int R, RS, rsl, Qt;  // rank, rank stride (power of two), its log2, tokens per chunk
  int nc, nT, NT, PT, nrb;
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

// The same product when both operands run along k in memory: A[m][k] at
// a[m * am + k] and B[k][n] at bt[n * bn + k], K a multiple of 16, 16-byte
// aligned rows.  Lane group q takes k = 16 j + 4 q + e in step (j, e), so
// each lane reads its operands as 16-byte vectors; A and B agree on the
// order, which the sum over k does not see.
__device__ __forceinline__ floatx4 mm_tile_k4(const float* a, int am, const float* bt, int bn, int K,
                                              floatx4 acc, int lane) {
  const int r = lane & 15, q = lane >> 4;
  const float* ap = a + r * am + 4 * q;
  const float* bq = bt + r * bn + 4 * q;
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 16) {
    const floatx4 av = lds_read4(ap + k0), bv = lds_read4(bq + k0);
    acc = mfma16(av[0], bv[0], acc);
    acc = mfma16(av[1], bv[1], acc);
    acc = mfma16(av[2], bv[2], acc);
    acc = mfma16(av[3], bv[3], acc);
  }
  return acc;
}

// A from LDS along k as in mm_tile_k4; B[k][n] = g[n * ldg + k] from global
// memory, rows clamped to nrow - 1 and k to kmax - 4 (N % 4 == 0), so reads
// stay in bounds; A is zero where k runs past the data, and clamped rows give
// output columns the caller discards.  All B loads are issued first.
template <int KMAX16>
__device__ __forceinline__ floatx4 mm_tile_k4_g(const float* a, int am, const float* g, int ldg, int nrow,
                                                int kmax, int K, floatx4 acc, int lane) {
  const int r = lane & 15, q = lane >> 4;
  const float* ap = a + r * am + 4 * q;
  const float* gp = g + (size_t)min(r, nrow - 1) * ldg;
  floatx4 bv[KMAX16];
#pragma unroll
  for (int j = 0; j < KMAX16; ++j)
    if (16 * j < K) bv[j] = *reinterpret_cast<const floatx4*>(gp + min(16 * j + 4 * q, kmax - 4));
#pragma unroll
  for (int j = 0; j < KMAX16; ++j) {
    if (16 * j < K) {
      const floatx4 av = lds_read4(ap + 16 * j);
      acc = mfma16(av[0], bv[j][0], acc);
      acc = mfma16(av[1], bv[j][1], acc);
      acc = mfma16(av[2], bv[j][2], acc);
      acc = mfma16(av[3], bv[j][3], acc);
    }
  }
  return acc;
}

// The same product for any N: scalar loads, k = 4 j + q in step j.
template <int KMAX4>
__device__ __forceinline__ floatx4 mm_tile_k1_g(const float* a, int am, const float* g, int ldg, int nrow,
                                                int kmax, int K, floatx4 acc, int lane) {
  const int r = lane & 15, q = lane >> 4;
  const float* ap = a + r * am + q;
  const float* gp = g + (size_t)min(r, nrow - 1) * ldg;
  float bv[KMAX4];
#pragma unroll
  for (int j = 0; j < KMAX4; ++j)
    if (4 * j < K) bv[j] = gp[min(4 * j + q, kmax - 1)];
#pragma unroll
  for (int j = 0; j < KMAX4; ++j)
    if (4 * j < K) acc = mfma16(ap[4 * j], bv[j], acc);
  return acc;
}

// A[m][k] from LDS (a[m * am + k]); B[k][n] = g[k * ldg + n] from global
// memory, k clamped to krow - 1 and n to ncol - 1 (A is zero past krow; the
// caller discards output columns past ncol).  K a multiple of 4, at most 4 KMAX4.
template <int KMAX4>
__device__ __forceinline__ floatx4 mm_tile_g(const float* a, int am, const float* g, int ldg, int krow,
                                             int ncol, int K, floatx4 acc, int lane) {
  const int r = lane & 15, q = lane >> 4;
  const float* ap = a + r * am + q;
  const float* gp = g + min(r, ncol - 1);
  float bv[KMAX4];
#pragma unroll
  for (int j = 0; j < KMAX4; ++j)
    if (4 * j < K) bv[j] = gp[(size_t)min(4 * j + q, krow - 1) * ldg];
#pragma unroll
  for (int j = 0; j < KMAX4; ++j)
    if (4 * j < K) acc = mfma16(ap[4 * j], bv[j], acc);
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

// Inclusive suffix sum within each aligned group of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float suffix_sum(float v, int lane) {
#pragma unroll
  for (int off = 1; off < W; off <<= 1) {
    const float o = __shfl_down(v, off, W);
    if ((lane & (W - 1)) + off < W) v += o;
  }
  return v;
}

__device__ __forceinline__ float theta_at(const BwdK& p, int bh, int t, int a) {
  return p.theta[((size_t)bh * p.L + t) * p.A + a] + p.tpre[((size_t)bh * p.nT + t / TT) * p.A + a];
}

// Rotated, bias-added keys and queries of one chunk into LDS rows of stride
// ns (columns N .. 16 NT - 1 and rows past nv zero); with cs / sn non-null
// also the cosines and sines [BQ][A].  Column j < A pairs with j + A;
// A <= j < N - A stands for the plain column j + A.  All loads of a thread
// of a round of KQ_ROUND items are issued before the first is used (clamped
// in-range indices).
__device__ void load_kq(const BwdK& p, int b, int h, int g, int t0, int nv, float* Kc, float* Qc, int ns,
                        float* cs_l, float* sn_l, int tid) {
  const int N = p.N, A = p.A, NP = N - A, bh = b * p.H + h;
  const float* bb = p.b_bias + (size_t)h * N;
  const float* cb = p.c_bias + (size_t)h * N;
  for (int k0 = 0; k0 < KQ_ITEMS && 512 * k0 < BQ * NP; k0 += KQ_ROUND) {
  float th[KQ_ROUND], b0[KQ_ROUND], b1[KQ_ROUND], c0[KQ_ROUND], c1[KQ_ROUND];
  float bb0[KQ_ROUND], bb1[KQ_ROUND], cb0[KQ_ROUND], cb1[KQ_ROUND];
#pragma unroll
  for (int kk = 0; kk < KQ_ROUND; ++kk) {
    const int k = kk;
    const int it = min(tid + 512 * (k0 + kk), BQ * NP - 1);
    const int t = it / NP, j = it - t * NP;
    const int tc = t0 + min(t, nv - 1);
    const int n0 = j < A ? j : j + A;
    const int n1 = j < A ? j + A : n0;
    const size_t row = (((size_t)b * p.L + tc) * p.G + g) * N;
    th[k] = A > 0 ? theta_at(p, bh, tc, min(j, A - 1)) : 0.f;
    b0[k] = p.b[row + n0]; b1[k] = p.b[row + n1];
    c0[k] = p.c[row + n0]; c1[k] = p.c[row + n1];
    bb0[k] = bb[n0]; bb1[k] = bb[n1];
    cb0[k] = cb[n0]; cb1[k] = cb[n1];
  }
#pragma unroll
  for (int k = 0; k < KQ_ROUND; ++k) {
    const int it = tid + 512 * (k0 + k);
    if (it >= BQ * NP) break;
    const int t = it / NP, j = it - t * NP;
    const bool ok = t < nv;
    if (j < A) {
      float sn, cs;
      sincos_acc(th[k], &sn, &cs);
      const float kb0 = b0[k] + bb0[k], kb1 = b1[k] + bb1[k];
      const float qc0 = c0[k] + cb0[k], qc1 = c1[k] + cb1[k];
      Kc[t * ns + j] = ok ? kb0 * cs - kb1 * sn : 0.f;
      Kc[t * ns + j + A] = ok ? kb0 * sn + kb1 * cs : 0.f;
      Qc[t * ns + j] = ok ? qc0 * cs - qc1 * sn : 0.f;
      Qc[t * ns + j + A] = ok ? qc0 * sn + qc1 * cs : 0.f;
      if (cs_l) {
        cs_l[t * A + j] = cs;
        sn_l[t * A + j] = sn;
      }
    } else {
      Kc[t * ns + j + A] = ok ? b0[k] + bb0[k] : 0.f;
      Qc[t * ns + j + A] = ok ? c0[k] + cb0[k] : 0.f;
    }
  }
  }
  const int pad = p.NT * 16 - N;  // zero columns N .. 16 NT - 1
  for (int it = tid; it < BQ * pad; it += 512) {
    const int t = it / pad, n = N + (it - t * pad);
    Kc[t * ns + n] = 0.f;
    Qc[t * ns + n] = 0.f;
  }
}

// x and gy = dout * silu(z) of one chunk into LDS rows of stride ps (zero
// past nv and P); with wx non-null, row t of x is scaled by wx[t] and row t
// of gy by wg[t].  Loads first, then the stores.
__device__ void load_xg(const BwdK& p, int b, int h, int t0, int nv, float* X, float* GY, int ps,
                        const float* wx, const float* wg, int tid) {
  const int P = p.P, PP = p.PT * 16;
  float xv[XG_ITEMS], gv[XG_ITEMS], zv[XG_ITEMS];
#pragma unroll
  for (int k = 0; k < XG_ITEMS; ++k) {
    const int it = min(tid + 512 * k, BQ * PP - 1);
    const int t = it / PP, pp = it - t * PP;
    const size_t gi = (((size_t)b * p.L + t0 + min(t, nv - 1)) * p.H + h) * P + min(pp, P - 1);
    xv[k] = p.x[gi];
    gv[k] = p.dout[gi];
    zv[k] = p.has_z ? p.z[gi] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < XG_ITEMS; ++k) {
    const int it = tid + 512 * k;
    if (it >= BQ * PP) break;
    const int t = it / PP, pp = it - t * PP;
    const bool ok = t < nv && pp < P;
    float gy = gv[k];
    if (p.has_z) gy *= siluf_acc(zv[k]);
    float x = xv[k];
    if (wx) {
      x *= wx[t];
      gy *= wg[t];
    }
    X[t * ps + pp] = ok ? x : 0.f;
    GY[t * ps + pp] = ok ? gy : 0.f;
  }
}

// Chunk geometry: state size N, head_dim P, angle count A and their 16-wide
// tile counts.  The specialised kernels fix them at compile time (NC > 0), so
// index division and loop bounds fold to constants.
struct Geom {
  int N, P, A, NT, PT;
};

template <int NC, int PC, int AC>
__device__ __forceinline__ Geom geom_of(const BwdK& p) {
  if constexpr (NC > 0)
    return Geom{NC, PC, AC, (NC + 15) / 16, (PC + 15) / 16};
  else
    return Geom{p.N, p.P, p.A, p.NT, p.PT};
}

__device__ __forceinline__ floatx4 ldg4(const float* q) { return *reinterpret_cast<const floatx4*>(q); }
__device__ __forceinline__ void sts4(float* q, floatx4 v) { *reinterpret_cast<floatx4*>(q) = v; }

__device__ __forceinline__ float dsilu_fast(float u) {
  const float s = sigmoid_fast(u);
  return s * (1.f + u * (1.f - s));
}

// load_kq with 16-byte accesses, for N and A multiples of 4, N a multiple of
// 16 (no pad columns), 16-byte aligned operand rows and LDS rows.  An item is
// four columns of one token: the first BQ A / 4 threads take the rotated
// pairs (columns j .. j + 3 with their partners j + A ..), then all threads
// share the plain columns 2 A .. N - 1; branches are wave-uniform when
// BQ A / 4 is a multiple of 64.  Row offsets within the chunk are 32-bit.
__device__ __forceinline__ void load_kq4(const BwdK& p, const Geom gm, int b, int h, int g, int t0, int nv,
                                         float* Kc, float* Qc, int ns, float* cs_l, float* sn_l, int tid) {
  const int N = gm.N, A = gm.A, A4 = A / 4, NP4 = (N - 2 * A) / 4;
  const int bh = b * p.H + h, GN = p.G * N;
  const size_t row0 = ((size_t)b * p.L + t0) * GN + (size_t)g * N;
  const float* brow = p.b + row0;  // token t0 + t, column n at brow[t * GN + n]
  const float* crow = p.c + row0;
  const float* bb = p.b_bias + (size_t)h * N;
  const float* cb = p.c_bias + (size_t)h * N;
  if (A > 0) {
    const float* th = p.theta + ((size_t)bh * p.L + t0) * A;
    const float* tp = p.tpre + ((size_t)bh * p.nT + t0 / TT) * A;  // a chunk lies inside one tile
    for (int it = tid; it < BQ * A4; it += 512) {
      const int t = it / A4, j = 4 * (it - t * A4);
      const int tc = min(t, nv - 1), ro = tc * GN;
      const floatx4 th4 = ldg4(th + tc * A + j), tp4 = ldg4(tp + j);
      const floatx4 b0 = ldg4(brow + ro + j), b1 = ldg4(brow + ro + j + A);
      const floatx4 c0 = ldg4(crow + ro + j), c1 = ldg4(crow + ro + j + A);
      const floatx4 bb0 = ldg4(bb + j), bb1 = ldg4(bb + j + A), cb0 = ldg4(cb + j), cb1 = ldg4(cb + j + A);
      const bool ok = t < nv;
      floatx4 k0, k1, q0, q1, cs4, sn4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sn, cs;
        sincos_acc(th4[e] + tp4[e], &sn, &cs);
        const float kb0 = b0[e] + bb0[e], kb1 = b1[e] + bb1[e];
        const float qc0 = c0[e] + cb0[e], qc1 = c1[e] + cb1[e];
        k0[e] = ok ? kb0 * cs - kb1 * sn : 0.f;
        k1[e] = ok ? kb0 * sn + kb1 * cs : 0.f;
        q0[e] = ok ? qc0 * cs - qc1 * sn : 0.f;
        q1[e] = ok ? qc0 * sn + qc1 * cs : 0.f;
        cs4[e] = cs;
        sn4[e] = sn;
      }
      sts4(Kc + t * ns + j, k0);
      sts4(Kc + t * ns + j + A, k1);
      sts4(Qc + t * ns + j, q0);
      sts4(Qc + t * ns + j + A, q1);
      if (cs_l) {
        sts4(cs_l + t * A + j, cs4);
        sts4(sn_l + t * A + j, sn4);
      }
    }
  }
  for (int it = tid; it < BQ * NP4; it += 512) {
    const int t = it / NP4, n = 2 * A + 4 * (it - t * NP4);
    const int tc = min(t, nv - 1), ro = tc * GN;
    const floatx4 b4 = ldg4(brow + ro + n), c4 = ldg4(crow + ro + n);
    const floatx4 bb4 = ldg4(bb + n), cb4 = ldg4(cb + n);
    const bool ok = t < nv;
    floatx4 kv, qv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[e] = ok ? b4[e] + bb4[e] : 0.f;
      qv[e] = ok ? c4[e] + cb4[e] : 0.f;
    }
    sts4(Kc + t * ns + n, kv);
    sts4(Qc + t * ns + n, qv);
  }
}

// load_xg with 16-byte accesses, for P a multiple of 16 (no pad columns) and
// 16-byte aligned rows: item (token, four head_dim columns).
__device__ __forceinline__ void load_xg4(const BwdK& p, const Geom gm, int b, int h, int t0, int nv, float* X,
                                         float* GY, int ps, const float* wx, const float* wg, int tid) {
  const int P = gm.P, P4 = P / 4, HP = p.H * P;
  const size_t row0 = (((size_t)b * p.L + t0) * p.H + h) * P;  // token t0 + t at row0 + t * HP
  for (int it = tid; it < BQ * P4; it += 512) {
    const int t = it / P4, pp = 4 * (it - t * P4);
    const int o = min(t, nv - 1) * HP + pp;
    const floatx4 x4 = ldg4(p.x + row0 + o), g4 = ldg4(p.dout + row0 + o);
    const floatx4 z4 = p.has_z ? ldg4(p.z + row0 + o) : floatx4{0.f, 0.f, 0.f, 0.f};
    const bool ok = t < nv;
    const float sx = wx ? wx[t] : 1.f, sg = wg ? wg[t] : 1.f;
    floatx4 xv, gv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gy = p.has_z ? g4[e] * silu_fast(z4[e]) : g4[e];
      xv[e] = ok ? x4[e] * sx : 0.f;
      gv[e] = ok ? gy * sg : 0.f;
    }
    sts4(X + t * ps + pp, xv);
    sts4(GY + t * ps + pp, gv);
  }
}

// (1) Cumulative angle within each 64-token tile and the tile totals; one wave
// per (b, h, tile), lane a < A.
__global__ __launch_bounds__(64) void bwd_theta_local_kernel(BwdK p) {
  __shared__ float dts[TT];
  __shared__ float angs[TT * 65];
  const int bh = blockIdx.x / p.nT, tile = blockIdx.x - bh * p.nT;
  const int b = bh / p.H, h = bh - b * p.H, A = p.A, L = p.L;
  const int lane = threadIdx.x;
  const int t0 = tile * TT, nv = min(TT, L - t0);
  dts[lane] = lane < nv ? p.dt[((size_t)b * L + t0 + lane) * p.H + h] : 0.f;
  for (int i = lane; i < TT * A; i += 64) {
    const int t = i / A, a = i - t * A;
    angs[t * 65 + a] = t < nv ? p.angle[((size_t)b * L + t0 + t) * A + a] : 0.f;
  }
  __syncthreads();
  if (lane >= A) return;
  float run = 0.f;
  float* out = p.theta + ((size_t)bh * L + t0) * A + lane;
  for (int t = 0; t < nv; ++t) {
    run = fmaf(dts[t], angs[t * 65 + lane], run);
    out[(size_t)t * A] = run;
  }
  p.tpre[((size_t)bh * p.nT + tile) * A + lane] = run;
}

// (1) for A <= 32: one wave per (b, h, tile), half-wave e over tokens
// 32 e .. 32 e + 31 of the tile and lane a < 32 over the angles; the angles
// are read straight from global memory (a 128-byte row per token), dt
// travels between lanes, and the second half adds the first half's total.
__global__ __launch_bounds__(64) void bwd_theta_local32_kernel(BwdK p) {
  const int bh = blockIdx.x / p.nT, tile = blockIdx.x - bh * p.nT;
  const int b = bh / p.H, h = bh - b * p.H, A = p.A, L = p.L;
  const int lane = threadIdx.x, a = lane & 31, e = lane >> 5;
  const int t0 = tile * TT, nv = min(TT, L - t0);
  const float dtv = lane < nv ? p.dt[((size_t)b * L + t0 + lane) * p.H + h] : 0.f;  // lane = token
  const bool col = a < A;
  const float* ang = p.angle + ((size_t)b * L + t0 + 32 * e) * A + min(a, A - 1);
  float th[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) th[i] = (col && 32 * e + i < nv) ? ang[i * A] : 0.f;
  float run = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    run = fmaf(__shfl(dtv, 32 * e + i, 64), th[i], run);
    th[i] = run;
  }
  const float first = __shfl(run, a, 64);  // the first half's total for angle a
  const float add = e ? first : 0.f;
  float* out = p.theta + ((size_t)bh * L + t0 + 32 * e) * A + a;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (col && 32 * e + i < nv) out[i * A] = th[i] + add;
  if (e == 1 && col) p.tpre[((size_t)bh * p.nT + tile) * A + a] = run + add;
}

// (2) Exclusive prefix over the tiles of the tile totals, in place; one wave
// per (b, h, a), lanes over tiles.
__global__ __launch_bounds__(64) void bwd_theta_scan_kernel(BwdK p) {
  const int bh = blockIdx.x / p.A, a = blockIdx.x - bh * p.A;
  const int lane = threadIdx.x;
  float carry = 0.f;
  for (int base = 0; base < p.nT; base += 64) {
    const int tile = base + lane;
    float* slot = p.tpre + ((size_t)bh * p.nT + tile) * p.A + a;
    const float v = tile < p.nT ? *slot : 0.f;
    // inclusive prefix over the 64 lanes
    float s = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(s, off, 64);
      if (lane >= off) s += o;
    }
    if (tile < p.nT) *slot = carry + s - v;
    carry += __shfl(s, 63, 64);
  }
}

// Per-token scalars of a chunk into LDS (wave 0, lanes 0..31 own the tokens):
// cum (inclusive chunk-local sum of adt), s, gamma, e^cum and e^(cumx - cum).
// Tokens past the end get adt = s = gamma = 0, so cum stays flat there.
struct ChunkScalars {
  float *cum, *scl, *gam, *ec, *ex;
};

__device__ void chunk_scalars(const BwdK& p, int b, int h, int t0, int nv, const ChunkScalars& cs, int lane) {
  const int t = t0 + min(lane & 31, nv - 1);
  const size_t i = ((size_t)b * p.L + t) * p.H + h;
  const bool has_next = t + 1 < p.L;
  const size_t i1 = has_next ? i + p.H : i;
  const float adt_r = p.adt[i], dt_r = p.dt[i], tr_r = p.trap[i], dt1 = p.dt[i1], tr1 = p.trap[i1];
  const bool ok = lane < nv;
  const float adt = ok ? adt_r : 0.f;
  const float gam = ok ? sigmoidf_acc(tr_r) * dt_r : 0.f;
  const float s = ok ? gam + (has_next ? (1.f - sigmoidf_acc(tr1)) * dt1 : 0.f) : 0.f;
  const float cum = scan32_f(lane < 32 ? adt : 0.f);
  const float cumx = __shfl(cum, 31, 64);
  if (lane < BQ) {
    cs.cum[lane] = cum;
    cs.scl[lane] = s;
    cs.gam[lane] = gam;
    cs.ec[lane] = expf(cum);
    cs.ex[lane] = expf(cumx - cum);
  }
}

// (3) Per chunk: S = sum_s e^(cumx-cum_s) s_s x_s K_s^T and
// R = sum_r e^(cum_r) gy_r Q_r^T, both [P][N], and the chunk decay e^cumx.
// NC > 0: geometry fixed at (NC, PC, AC) with the 16-byte loaders.
template <int NC, int PC, int AC>
__global__ __launch_bounds__(512) void bwd_summary_kernel(BwdK p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const Geom gm = geom_of<NC, PC, AC>(p);
  const int NS = gm.NT * 16 + 4, PS = gm.PT * 16 + 4, P = gm.P, N = gm.N;
  float* Kc = lds;
  float* Qc = Kc + BQ * NS;
  float* Xw = Qc + BQ * NS;
  float* Gw = Xw + BQ * PS;
  float* cum = Gw + BQ * PS;
  float* scl = cum + BQ;
  float* gam = scl + BQ;
  float* ec = gam + BQ;
  float* ex = ec + BQ;
  float* wx = ex + BQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int bh = blockIdx.x / p.nc, c = blockIdx.x - bh * p.nc;
  const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
  const int t0 = c * BQ, nv = min(BQ, p.L - t0);
  if (wave == 0) chunk_scalars(p, b, h, t0, nv, ChunkScalars{cum, scl, gam, ec, ex}, lane);
  if constexpr (NC > 0)
    load_kq4(p, gm, b, h, g, t0, nv, Kc, Qc, NS, nullptr, nullptr, tid);
  else
    load_kq(p, b, h, g, t0, nv, Kc, Qc, NS, nullptr, nullptr, tid);
  __syncthreads();
  if (tid < BQ) wx[tid] = ex[tid] * scl[tid];
  __syncthreads();
  if constexpr (NC > 0)
    load_xg4(p, gm, b, h, t0, nv, Xw, Gw, PS, wx, ec, tid);
  else
    load_xg(p, b, h, t0, nv, Xw, Gw, PS, wx, ec, tid);
  __syncthreads();
  if (tid == 0) p.decay[blockIdx.x] = expf(cum[BQ - 1]);
  const int ntile = gm.PT * gm.NT;
  const size_t base = (size_t)blockIdx.x * P * N;
  const int r = lane & 15, q = lane >> 4;
  for (int job = wave; job < 2 * ntile; job += nw) {
    const bool rev = job >= ntile;
    const int jt = rev ? job - ntile : job;
    const int pt = jt / gm.NT, nt = jt - pt * gm.NT;
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
      if (pp < P && n < N) dst[pp * N + n] = acc[i];
    }
  }
}

// (4) Element-wise over the chunks of one (b, h): hs[c] <- state before chunk
// c; gs[c] <- adjoint after chunk c.  In place; loads run U chunks ahead.
// mode 1: forward summaries (hs); 2: reverse summaries (gs); 3: both, one
// direction per blockIdx.y.  A thread owns V consecutive elements (V = 4:
// 16-byte accesses, P N a multiple of 4 and 16-byte aligned summaries).
template <int V>
__global__ __launch_bounds__(256) void bwd_prefix_kernel(BwdK p, int blocks_per_bh, int mode) {
  typedef float vec __attribute__((ext_vector_type(V)));
  const int bh = blockIdx.x / blocks_per_bh;
  const int e = ((blockIdx.x - bh * blocks_per_bh) * blockDim.x + threadIdx.x) * V;
  const int PN = p.P * p.N, nc = p.nc;
  if (e >= PN) return;
  const bool rev = mode == 2 || (mode == 3 && blockIdx.y == 1);
  float* base = (rev ? p.gs : p.hs) + (size_t)bh * nc * PN + e;
  const float* dec = p.decay + (size_t)bh * nc;
  constexpr int U = 8;
  vec run = (vec)0.f;
  for (int i0 = 0; i0 < nc; i0 += U) {
    vec v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = rev ? nc - 1 - (i0 + u) : i0 + u;
      v[u] = i0 + u < nc ? *reinterpret_cast<const vec*>(base + (size_t)c * PN) : (vec)0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u < nc) {
        const int c = rev ? nc - 1 - (i0 + u) : i0 + u;
        *reinterpret_cast<vec*>(base + (size_t)c * PN) = run;
        const float dc = dec[c];
#pragma unroll
        for (int l = 0; l < V; ++l) run[l] = fmaf(dc, run[l], v[u][l]);
      }
    }
  }
}

struct ChunkLds {
  int NS, PS;
  int o_kc, o_qc, o_x, o_gy, o_mqk, o_vv, o_msg, o_cs, o_sn, o_sc, o_part, total;
};

// x and gy, dead once the products are done, make room for staging one of
// dQ / dK [BQ][NS]; the masks make room for d theta [BQ][A].
__host__ __device__ inline ChunkLds chunk_lds(int PT, int NT, int A) {
  ChunkLds l{};
  l.NS = NT * 16 + 4;
  l.PS = PT * 16 + 4;
  int off = 0;
  l.o_kc = off; off += BQ * l.NS;
  l.o_qc = off; off += BQ * l.NS;
  l.o_x = off;
  l.o_gy = off + BQ * l.PS;
  off += 2 * BQ * l.PS > BQ * l.NS ? 2 * BQ * l.PS : BQ * l.NS;
  l.o_mqk = off; off += BQ * MS;
  l.o_vv = off; off += BQ * MS;
  l.o_msg = off; off += BQ * MS;
  l.o_cs = off; off += BQ * A;
  l.o_sn = off; off += BQ * A;
  l.o_sc = off; off += 7 * BQ;
  l.o_part = off; off += 2 * BQ * PT;
  l.total = off;
  return l;
}

// (5) Per chunk: y, GK, dQ, dK on FP32 MFMA; writes d_z, d_x, the per-head
// adjoints of B + b_bias and C + c_bias, and the chunk-local suffix sums of
// the d adt terms (into d_adt) and of d theta, with their chunk totals.
// NC > 0: geometry fixed at (NC, PC, AC) = (16 x 8 waves, multiple of 16,
// multiple of 4 with BQ AC / 4 a multiple of 64), 16-byte loaders and stores,
// and each wave reuses its state columns for both token halves of dQ and dK.
template <bool VEC4, int NC, int PC, int AC>
__global__ __launch_bounds__(512, 4) void bwd_chunk_kernel(BwdK p) {
  constexpr bool FIX = NC > 0;
  static_assert(!FIX || (NC == 128 && PC % 16 == 0 && AC % 4 == 0 && (BQ * AC / 4) % 64 == 0),
                "fixed geometry: N = 128 (one state tile per wave), P a multiple of 16");
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const Geom gm = geom_of<NC, PC, AC>(p);
  const ChunkLds ll = chunk_lds(gm.PT, gm.NT, gm.A);
  const int NS = ll.NS, PS = ll.PS, PP = gm.PT * 16, NN = gm.NT * 16;
  float* Kc = lds + ll.o_kc;
  float* Qc = lds + ll.o_qc;
  float* X = lds + ll.o_x;
  float* GY = lds + ll.o_gy;
  float* MQK = lds + ll.o_mqk;
  float* VV = lds + ll.o_vv;
  float* MSG = lds + ll.o_msg;
  float* CS = lds + ll.o_cs;
  float* SN = lds + ll.o_sn;
  float* cum = lds + ll.o_sc;
  float* scl = cum + BQ;
  float* gam = scl + BQ;
  float* ec = gam + BQ;
  float* ex = ec + BQ;
  float* qk = ex + BQ;
  float* xg = qk + BQ;
  float* rho_part = lds + ll.o_part;        // [BQ][PT]
  float* ds_part = rho_part + BQ * gm.PT;   // [BQ][PT]
  float* STG = X;                           // after the products: dQ, then dK [BQ][NS]
  float* DTH = MQK;                         // after the products: d theta [BQ][A]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / p.nc, c = blockIdx.x - bh * p.nc;
  const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
  const int t0 = c * BQ, nv = min(BQ, p.L - t0);
  const int P = gm.P, N = gm.N, H = p.H, A = gm.A, NP = N - A;
  const int HP = H * P;
  const size_t xrow0 = (((size_t)b * p.L + t0) * H + h) * P;  // token t0 + t, column pp at xrow0 + t HP + pp

  // ---- loads: keys/queries, x/gy, scalars (the state and adjoint tiles are
  // read from global memory by the products that use them)
  const float* HEg = p.hs + (size_t)blockIdx.x * P * N;  // h'_e [P][N]
  const float* GXg = p.gs + (size_t)blockIdx.x * P * N;  // G_x [P][N]
  // VEC4: N % 4 == 0, 16-byte rows: vector loads of the state rows
  if (wave == 0) chunk_scalars(p, b, h, t0, nv, ChunkScalars{cum, scl, gam, ec, ex}, lane);
  if constexpr (FIX) {
    load_kq4(p, gm, b, h, g, t0, nv, Kc, Qc, NS, CS, SN, tid);
    load_xg4(p, gm, b, h, t0, nv, X, GY, PS, nullptr, nullptr, tid);
  } else {
    load_kq(p, b, h, g, t0, nv, Kc, Qc, NS, CS, SN, tid);
    load_xg(p, b, h, t0, nv, X, GY, PS, nullptr, nullptr, tid);
  }
  const int r = lane & 15, q = lane >> 4;
  // fixed geometry: this wave's state tile (read by the y / G K products
  // below) loads now, during the staging and the chunk-square products
  floatx4 sv[FIX ? NC / 16 : 1];
  if constexpr (FIX) {
    const float* Sg = (wave >= 4 ? GXg : HEg) + ((wave & 3) * 16 + r) * N + 4 * q;  // B[k][n] = S[pt 16 + n][k]
#pragma unroll
    for (int j = 0; j < NC / 16; ++j) sv[j] = ldg4(Sg + 16 * j);
  }
  __syncthreads();
  const float Dh = p.has_d ? p.d[h] : 0.f;

  // ---- chunk-square products, masked: waves 0-3 Q K^T, waves 4-7 gy x^T
  {
    const bool sgx = wave >= 4;
    const int mt = (wave & 3) >> 1, st = wave & 1;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!sgx)
      acc = mm_tile_k4(Qc + mt * 16 * NS, NS, Kc + st * 16 * NS, NS, NN, acc, lane);
    else
      acc = mm_tile_k4(GY + mt * 16 * PS, PS, X + st * 16 * PS, PS, PP, acc, lane);
    const int s = st * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = mt * 16 + 4 * q + i;
      const float v = acc[i];
      const float dec = s < t ? (FIX ? exp_fast(cum[t] - cum[s]) : expf(cum[t] - cum[s])) : 0.f;
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

  // ---- y and GK (per head_dim tile), then dQ and dK (per state tile)
  const int nY = 2 * gm.PT, nQ = 2 * gm.NT;
  if constexpr (FIX) {
    // wave w: y (w < 4) or G K (w >= 4) for head_dim tile pt = w & 3 and both
    // token halves, so each state tile is read from global memory once
    const bool isgk = wave >= 4;
    const int pt = wave & 3;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
      const float* ap = (isgk ? Kc : Qc) + (mt * 16 + r) * NS + 4 * q;
#pragma unroll
      for (int j = 0; j < NC / 16; ++j) {
        const floatx4 av = lds_read4(ap + 16 * j);
        a1 = mfma16(av[0], sv[j][0], a1);
        a1 = mfma16(av[1], sv[j][1], a1);
        a1 = mfma16(av[2], sv[j][2], a1);
        a1 = mfma16(av[3], sv[j][3], a1);
      }
      if (!isgk)
        a2 = mm_tile(MQK + mt * 16 * MS, MS, 1, X + pt * 16, PS, 1, BQ, a2, lane);
      else
        a2 = mm_tile(VV + mt * 16, 1, MS, GY + pt * 16, PS, 1, BQ, a2, lane);
      const int pp = pt * 16 + r;
      float zv[4], gov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + 4 * q + i;
        const int o = min(t, nv - 1) * HP + min(pp, P - 1);
        zv[i] = (!isgk && p.has_z) ? p.z[xrow0 + o] : 0.f;
        gov[i] = (!isgk && p.has_z) ? p.dout[xrow0 + o] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + 4 * q + i;
        const bool ok = t < nv && pp < P;
        const size_t gi = xrow0 + t * HP + pp;
        const float xv = X[t * PS + pp], gy = GY[t * PS + pp];
        float part;
        if (!isgk) {
          const float y = fmaf(ec[t], a1[i], a2[i]);
          part = gy * y;
          if (ok) p.d_z[gi] = p.has_z ? gov[i] * fmaf(Dh, xv, y) * (FIX ? dsilu_fast(zv[i]) : dsilu_acc(zv[i])) : 0.f;
        } else {
          const float gk = fmaf(ex[t], a1[i], a2[i]);
          part = xv * gk;
          if (ok) p.d_x[gi] = fmaf(Dh + gam[t] * qk[t], gy, scl[t] * gk);
        }
        part = row16_sum(ok ? part : 0.f);
        if (r == 15) (isgk ? ds_part : rho_part)[t * gm.PT + pt] = part;
      }
    }
  } else {
    for (int job = wave; job < 2 * nY; job += 8) {
      const bool isgk = job >= nY;
      const int jj = isgk ? job - nY : job;
      const int mt = jj / gm.PT, pt = jj - mt * gm.PT;
      floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
      const float* Sg = (isgk ? GXg : HEg) + (size_t)pt * 16 * N;
      const int prow = P - pt * 16;
      const float* Ra = (isgk ? Kc : Qc) + mt * 16 * NS;
      if constexpr (VEC4)
        a1 = mm_tile_k4_g<8>(Ra, NS, Sg, N, prow, N, NN, a1, lane);
      else
        a1 = mm_tile_k1_g<32>(Ra, NS, Sg, N, prow, N, NN, a1, lane);
      if (!isgk)
        a2 = mm_tile(MQK + mt * 16 * MS, MS, 1, X + pt * 16, PS, 1, BQ, a2, lane);
      else
        a2 = mm_tile(VV + mt * 16, 1, MS, GY + pt * 16, PS, 1, BQ, a2, lane);
      const int pp = pt * 16 + r;
      float zv[4], gov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + 4 * q + i;
        const int o = min(t, nv - 1) * HP + min(pp, P - 1);
        zv[i] = (!isgk && p.has_z) ? p.z[xrow0 + o] : 0.f;
        gov[i] = (!isgk && p.has_z) ? p.dout[xrow0 + o] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + 4 * q + i;
        const bool ok = t < nv && pp < P;
        const size_t gi = xrow0 + t * HP + pp;
        const float xv = X[t * PS + pp], gy = GY[t * PS + pp];
        float part;
        if (!isgk) {
          const float y = fmaf(ec[t], a1[i], a2[i]);
          part = gy * y;
          if (ok) p.d_z[gi] = p.has_z ? gov[i] * fmaf(Dh, xv, y) * (FIX ? dsilu_fast(zv[i]) : dsilu_acc(zv[i])) : 0.f;
        } else {
          const float gk = fmaf(ex[t], a1[i], a2[i]);
          part = xv * gk;
          if (ok) p.d_x[gi] = fmaf(Dh + gam[t] * qk[t], gy, scl[t] * gk);
        }
        part = row16_sum(ok ? part : 0.f);
        if (r == 15) (isgk ? ds_part : rho_part)[t * gm.PT + pt] = part;
      }
    }
  }
  floatx4 res[4];
  if constexpr (FIX) {
    // job k of wave w: state columns 16 w .. 16 w + 15, token half k & 1,
    // dQ (k < 2) or dK; the state columns are loaded once for both halves.
    const int nt = wave;
    float sh[PC / 4], sg[PC / 4];
#pragma unroll
    for (int j = 0; j < PC / 4; ++j) {
      sh[j] = HEg[(4 * j + q) * N + nt * 16 + r];
      sg[j] = GXg[(4 * j + q) * N + nt * 16 + r];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool isdk = k >= 2;
      const int mt = k & 1;
      floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
      const float* Ar = (isdk ? X : GY) + (mt * 16 + r) * PS + q;  // A[m=t][k=p]
#pragma unroll
      for (int j = 0; j < PC / 4; ++j) a1 = mfma16(Ar[4 * j], isdk ? sg[j] : sh[j], a1);
      if (!isdk)
        a2 = mm_tile(MSG + mt * 16 * MS, MS, 1, Kc + nt * 16, NS, 1, BQ, a2, lane);
      else
        a2 = mm_tile(MSG + mt * 16, 1, MS, Qc + nt * 16, NS, 1, BQ, a2, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = mt * 16 + 4 * q + i;
        const float w = isdk ? scl[t] * ex[t] : ec[t];
        res[k][i] = fmaf(w, a1[i], a2[i]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int job = wave + 8 * k;
      res[k] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (job < 2 * nQ) {
        const bool isdk = job >= nQ;
        const int jj = isdk ? job - nQ : job;
        const int mt = jj / gm.NT, nt = jj - mt * gm.NT;
        floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
        const float* Sg = (isdk ? GXg : HEg) + nt * 16;
        if (!isdk) {
          a1 = mm_tile_g<32>(GY + mt * 16 * PS, PS, Sg, N, P, N - nt * 16, PP, a1, lane);
          a2 = mm_tile(MSG + mt * 16 * MS, MS, 1, Kc + nt * 16, NS, 1, BQ, a2, lane);
        } else {
          a1 = mm_tile_g<32>(X + mt * 16 * PS, PS, Sg, N, P, N - nt * 16, PP, a1, lane);
          a2 = mm_tile(MSG + mt * 16, 1, MS, Qc + nt * 16, NS, 1, BQ, a2, lane);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = mt * 16 + 4 * q + i;
          const float w = isdk ? scl[t] * ex[t] : ec[t];
          res[k][i] = fmaf(w, a1[i], a2[i]);
        }
      }
    }
  }
  // ---- rotation adjoints, queries first, then keys: stage the adjoint tiles
  // in LDS, then d theta and the un-rotated adjoints per head
  const size_t hrow0 = (((size_t)b * p.L + t0) * H + h) * N;  // token t0 + t at hrow0 + t H N
  const int HN = H * N;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();  // x, gy, the masks (pass 0) or the staged dQ (pass 1) are free
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int job = wave + 8 * k;
      if (job < 2 * nQ && (job >= nQ) == (pass == 1)) {
        const int jj = pass ? job - nQ : job;
        const int mt = jj / gm.NT, nt = jj - mt * gm.NT;
#pragma unroll
        for (int i = 0; i < 4; ++i) STG[(mt * 16 + 4 * q + i) * NS + nt * 16 + r] = res[k][i];
      }
    }
    __syncthreads();
    const float* R = pass ? Kc : Qc;
    float* dst = (pass ? p.db_head : p.dc_head) + hrow0;
    if constexpr (FIX) {
      constexpr int A4 = AC / 4, NP4 = (NC - 2 * AC) / 4;
      for (int it = tid; it < BQ * A4; it += 512) {
        const int t = it / A4, j = 4 * (it - t * A4);
        if (t >= nv) {
          if (pass == 0) sts4(DTH + t * A + j, floatx4{0.f, 0.f, 0.f, 0.f});
          continue;
        }
        const floatx4 cs = lds_read4(CS + t * A + j), sn = lds_read4(SN + t * A + j);
        const floatx4 d0 = lds_read4(STG + t * NS + j), d1 = lds_read4(STG + t * NS + j + A);
        const floatx4 r0 = lds_read4(R + t * NS + j), r1 = lds_read4(R + t * NS + j + A);
        floatx4 th = pass ? lds_read4(DTH + t * A + j) : floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 u0, u1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = d1[e] * r0[e] - d0[e] * r1[e];
          th[e] = pass ? th[e] + v : v;
          u0[e] = d0[e] * cs[e] + d1[e] * sn[e];
          u1[e] = d1[e] * cs[e] - d0[e] * sn[e];
        }
        sts4(DTH + t * A + j, th);
        sts4(dst + t * HN + j, u0);
        sts4(dst + t * HN + j + A, u1);
      }
      for (int it = tid; it < BQ * NP4; it += 512) {
        const int t = it / NP4, n = 2 * AC + 4 * (it - t * NP4);
        if (t < nv) sts4(dst + t * HN + n, lds_read4(STG + t * NS + n));
      }
    } else {
      for (int it = tid; it < BQ * NP; it += 512) {
        const int t = it / NP, j = it - t * NP;
        if (t >= nv) {
          if (j < A && pass == 0) DTH[t * A + j] = 0.f;
          continue;
        }
        const int o = t * HN;
        if (j < A) {
          const float cs = CS[t * A + j], sn = SN[t * A + j];
          const float d0 = STG[t * NS + j], d1 = STG[t * NS + j + A];
          const float v = d1 * R[t * NS + j] - d0 * R[t * NS + j + A];
          DTH[t * A + j] = pass ? DTH[t * A + j] + v : v;
          dst[o + j] = d0 * cs + d1 * sn;
          dst[o + j + A] = d1 * cs - d0 * sn;
        } else {
          dst[o + j + A] = STG[t * NS + j + A];
        }
      }
    }
  }
  __syncthreads();

  // ---- chunk-local suffix sums
  if (wave == 0) {
    // d adt terms: rho_t - c_{t+1} ds_t - gamma_t e_t, with c_{t+1} = s_t - gamma_t
    float phi = 0.f, xgv = 0.f;
    if (lane < nv) {
      float rh = 0.f, ds = 0.f;
      for (int pt = 0; pt < gm.PT; ++pt) {
        rh += rho_part[lane * gm.PT + pt];
        ds += ds_part[lane * gm.PT + pt];
      }
      xgv = xg[lane];
      const float e = fmaf(xgv, qk[lane], ds);
      phi = rh - (scl[lane] - gam[lane]) * ds - gam[lane] * e;
      const size_t ri = (size_t)bh * p.L + t0 + lane;
      p.dsv[ri] = ds;
      p.ev[ri] = e;
    }
    const float loc = suffix_sum<32>(lane < 32 ? phi : 0.f, lane);
    if (lane < nv) p.d_adt[((size_t)b * p.L + t0 + lane) * H + h] = loc;
    if (lane == 0) p.phi_tot[blockIdx.x] = loc;
    const float tot = scan32_f(lane < 32 ? xgv : 0.f);
    if (lane == 31) p.dd_part[blockIdx.x] = tot;
  } else if (tid >= 64 && tid < 64 + A) {
    const int a = tid - 64;
    float s = 0.f;
    float* dst = p.dtheta + ((size_t)bh * p.L + t0) * A + a;
    for (int t = nv - 1; t >= 0; --t) {
      s += DTH[t * A + a];
      dst[t * A] = s;
    }
    p.th_tot[(size_t)blockIdx.x * A + a] = s;
  }
}

// (6) Exclusive suffix over the chunks of the chunk totals, in place: one wave
// per (b, h, column); column 0 is the d adt terms, 1 + a the angle a.
__global__ __launch_bounds__(64) void bwd_chunk_scan_kernel(BwdK p) {
  const int ncol = p.A + 1;
  const int bh = blockIdx.x / ncol, col = blockIdx.x - bh * ncol;
  const int lane = threadIdx.x, nc = p.nc;
  float carry = 0.f;
  for (int top = nc - 1; top >= 0; top -= 64) {
    const int cidx = top - 63 + lane;  // lanes cover chunks top-63 .. top
    float* slot = col == 0 ? p.phi_tot + (size_t)bh * nc + cidx
                           : p.th_tot + ((size_t)bh * nc + cidx) * p.A + (col - 1);
    const bool ok = cidx >= 0;
    const float v = ok ? *slot : 0.f;
    const float s = suffix_sum<64>(v, lane);
    if (ok) *slot = carry + s - v;
    carry += __shfl(s, 0, 64);
  }
}

// (7) Per 32-token tile of one (b, h): d adt += the later chunks' terms; the
// angle suffix theta_bar_t[a] = local suffix + later chunks; d dt, d trap and
// the per-head angle adjoint dt_t theta_bar_t (in place of the suffix).  A
// tile spans 32 / Qt chunks; each token reads the totals of its own chunk.
__global__ __launch_bounds__(256) void bwd_apply_kernel(BwdK p) {
  __shared__ float part[8][32];
  const int ntile = (p.L + 31) / 32;
  const int bh = blockIdx.x / ntile, tile = blockIdx.x - bh * ntile;
  const int b = bh / p.H, h = bh - b * p.H;
  const int tid = threadIdx.x, t = tid & 31, k = tid >> 5;
  const int A = p.A, H = p.H;
  const int tt = tile * 32 + t;
  const bool ok = tt < p.L;
  const int tc = min(tt, p.L - 1);
  const size_t ci = (size_t)bh * p.nc + tc / p.Qt;  // the token's chunk
  const size_t si = ((size_t)b * p.L + tc) * H + h;
  const float dtv = p.dt[si];
  // the token scalars are loaded with the angle terms, before the barrier
  const size_t ri = (size_t)bh * p.L + tc;
  float trv = 0.f, e = 0.f, dc = 0.f, dadt = 0.f, ptot = 0.f;
  if (k == 0) {
    trv = p.trap[si];
    e = p.ev[ri];
    dc = tc >= 1 ? p.dsv[ri - 1] : 0.f;
    dadt = p.d_adt[si];
    ptot = p.phi_tot[ci];
  }
  float* dth = p.dtheta + ((size_t)bh * p.L + tc) * A;
  const float* tht = p.th_tot + ci * A;
  const float* ang = p.angle + ((size_t)b * p.L + tc) * A;
  float acc = 0.f;
#pragma unroll 4
  for (int a = k; a < A; a += 8) {
    const float tb = dth[a] + tht[a];
    if (ok) dth[a] = dtv * tb;
    acc = fmaf(tb, ang[a], acc);
  }
  part[k][t] = acc;
  __syncthreads();
  if (k == 0 && ok) {
    float rot = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) rot += part[kk][t];
    const float lam = sigmoidf_acc(trv);
    p.d_adt[si] = dadt + ptot;
    p.d_dt[si] = fmaf(lam, e, fmaf(1.f - lam, dc, rot));
    p.d_trap[si] = lam * (1.f - lam) * dtv * (e - dc);
  }
}

// (8) Per block of RB token rows (b, t) and group g: d_b, d_c = sums of the
// per-head adjoints over the group's heads, and partial bias sums.  A row of
// per-head adjoints has R N columns (rank r, state n); item (hs, col) owns
// column col of heads hs, hs + nhs, ... for every row, so each bias sum has
// one owner.
__global__ __launch_bounds__(256) void bwd_group_kernel(BwdK p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int N = p.N, H = p.H, G = p.G, HG = H / G, R = p.R, RN = R * N;
  const int g = blockIdx.y, blk = blockIdx.x;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int nhs = max(1, nthr / RN);
  const int nact = min(nhs, HG);
  float* bacc = lds;                  // [2][HG][RN] bias sums of this block
  float* gsum = bacc + 2 * HG * RN;   // [nact][2][RN] group partials per head subset
  for (int i = tid; i < 2 * HG * RN; i += nthr) bacc[i] = 0.f;
  __syncthreads();
  const int rows = p.B * p.L;
  for (int rr = 0; rr < RB; ++rr) {
    const int row = blk * RB + rr;
    if (row >= rows) break;
    for (int it = tid; it < nact * RN; it += nthr) {
      const int hs = it / RN, col = it - hs * RN;
      float gb = 0.f, gc = 0.f;
      const size_t base = ((size_t)row * H + g * HG) * RN + col;
#pragma unroll 4
      for (int hh = hs; hh < HG; hh += nhs) {
        const float vb = p.db_head[base + (size_t)hh * RN];
        const float vc = p.dc_head[base + (size_t)hh * RN];
        gb += vb;
        gc += vc;
        bacc[hh * RN + col] += vb;
        bacc[(HG + hh) * RN + col] += vc;
      }
      gsum[(hs * 2) * RN + col] = gb;
      gsum[(hs * 2 + 1) * RN + col] = gc;
    }
    __syncthreads();
    for (int col = tid; col < RN; col += nthr) {
      float sb = 0.f, sc = 0.f;
      for (int k = 0; k < nact; ++k) {
        sb += gsum[(k * 2) * RN + col];
        sc += gsum[(k * 2 + 1) * RN + col];
      }
      const int r = col / N, n = col - r * N;
      const size_t o = ((size_t)row * R * G + r * G + g) * N + n;  // B / C row r G + g
      p.d_b[o] = sb;
      p.d_c[o] = sc;
    }
    __syncthreads();
  }
  for (int i = tid; i < 2 * HG * RN; i += nthr) {
    const int which = i / (HG * RN), rem = i - which * HG * RN;
    const int hh = rem / RN, col = rem - hh * RN;
    p.bias_part[(((size_t)blk * 2 + which) * H + g * HG + hh) * RN + col] = bacc[i];
  }
}

// (8) with 16-byte accesses (N % 4 == 0, 16-byte aligned d_b, d_c and per-head
// adjoints): item (head subset hs, four columns) sums heads hs, hs + nhs, ...
// of the group for each of the block's RB rows in registers, writes the
// per-head bias partial of those rows, and the head subsets meet in LDS in a
// fixed order for d_b / d_c.
__global__ __launch_bounds__(256) void bwd_group4_kernel(BwdK p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // [nhs][RB][C4] float4
  const int N = p.N, H = p.H, G = p.G, HG = H / G, R = p.R, RN = R * N, C4 = RN / 4;
  const int g = blockIdx.y, blk = blockIdx.x, tid = threadIdx.x;
  const int nhs = min(max(1, 256 / C4), HG);
  const int rows = p.B * p.L, row0 = blk * RB;
  for (int which = 0; which < 2; ++which) {
    const float* src = which ? p.dc_head : p.db_head;
    float* out = which ? p.d_c : p.d_b;
    for (int it = tid; it < nhs * C4; it += 256) {
      const int hs = it / C4, c4 = it - hs * C4;
      floatx4 gacc[RB];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) gacc[rr] = floatx4{0.f, 0.f, 0.f, 0.f};
      for (int hh = hs; hh < HG; hh += nhs) {
        const float* col = src + ((size_t)row0 * H + g * HG + hh) * RN + 4 * c4;  // row row0 + rr at + rr H RN
        floatx4 v[RB];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
          v[rr] = row0 + rr < rows ? ldg4(col + (size_t)rr * H * RN) : floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 bs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          bs += v[rr];
          gacc[rr] += v[rr];
        }
        sts4(p.bias_part + (((size_t)blk * 2 + which) * H + g * HG + hh) * RN + 4 * c4, bs);
      }
      if (nhs == 1) {
        const int cc = 4 * c4, r = cc / N, n = cc - r * N;
#pragma unroll
        for (int rr = 0; rr < RB; ++rr)
          if (row0 + rr < rows) sts4(out + ((size_t)(row0 + rr) * R * G + r * G + g) * N + n, gacc[rr]);
      } else {
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) sts4(lds + ((hs * RB + rr) * C4 + c4) * 4, gacc[rr]);
      }
    }
    if (nhs > 1) {
      __syncthreads();
      for (int it = tid; it < RB * C4; it += 256) {
        const int rr = it / C4, c4 = it - rr * C4;
        floatx4 s = lds_read4(lds + (rr * C4 + c4) * 4);
        for (int k = 1; k < nhs; ++k) s += lds_read4(lds + ((k * RB + rr) * C4 + c4) * 4);
        const int cc = 4 * c4, r = cc / N, n = cc - r * N;
        if (row0 + rr < rows) sts4(out + ((size_t)(row0 + rr) * R * G + r * G + g) * N + n, s);
      }
      __syncthreads();
    }
  }
}

// (9a) d_b_bias and d_c_bias: column sums of the group kernel's block
// partials [nrb][2][H][R N]; a workgroup of 16 waves takes 64 consecutive
// columns (lane = column), wave w the partial rows w, w + 16, ... in order,
// and the 16 wave sums are added in order.  The workgroups after the bias
// columns sum d_d over the chunks' partials the same way (lane = head).
__global__ __launch_bounds__(1024) void bwd_bias_kernel(BwdK p) {
  __shared__ float red[16][64];
  const int HN = p.H * p.R * p.N, ncol = 2 * HN, nbb = (ncol + 63) / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float s = 0.f;
  int out = -1;
  if ((int)blockIdx.x < nbb) {
    const int col = blockIdx.x * 64 + lane;
    if (col < ncol) {
      out = col;
      const float* src = p.bias_part + col;  // partial row k at + k 2 H R N
#pragma unroll 4
      for (int k = w; k < p.nrb; k += 16) s += src[(size_t)k * ncol];
    }
  } else {
    const int hh = ((int)blockIdx.x - nbb) * 64 + lane;
    if (hh < p.H) {
      out = ncol + hh;
      const int per = p.B * p.nc;
      if (p.has_d) {
        for (int k = w; k < per; k += 16) {
          const int bb = k / p.nc, cc = k - bb * p.nc;
          s += p.dd_part[((size_t)bb * p.H + hh) * p.nc + cc];
        }
      }
    }
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && out >= 0) {
    float t = red[0][lane];
    for (int k = 1; k < 16; ++k) t += red[k][lane];
    if (out < HN) p.d_b_bias[out] = t;
    else if (out < ncol) p.d_c_bias[out - HN] = t;
    else p.d_d[out - ncol] = t;
  }
}

// (9b) d_angle[b][t][a] = sum_h (per-head angle adjoint).
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

// ---------------------------------------------------------------------------
// MIMO backward.  A chunk holds BQ = 32 virtual rows v = t RS + r (token t,
// rank r; rows of padding ranks r >= R stay zero), Qt = BQ / RS tokens, as
// in the forward scan.  The state is shared by the ranks, so every formula
// above holds with x K^T replaced by the rank sum: the masks take the tokens
// of the two rows (all rank pairs of one token get lam dt), d gamma and the
// same-token terms sum over rank pairs, and d x sums mimo_x * dX_r over ranks.
// ---------------------------------------------------------------------------

// Keys / queries of the chunk's virtual rows into LDS (stride ns, zero rows
// and columns past the data); with cs_l the cosines / sines [BQ][A].
__device__ void load_kq_m(const BwdK& p, int b, int h, int g, int t0, int nv, float* Kc, float* Qc, int ns,
                          float* cs_l, float* sn_l, int tid, int nthr) {
  const int N = p.N, A = p.A, NP = N - A, bh = b * p.H + h, RG = p.R * p.G;
  for (int it = tid; it < BQ * NP; it += nthr) {
    const int v = it / NP, j = it - v * NP;
    const int t = v >> p.rsl, r = v & (p.RS - 1);
    const bool ok = t < nv && r < p.R;
    const int n0 = j < A ? j : j + A;
    float k0 = 0.f, k1 = 0.f, q0 = 0.f, q1 = 0.f, cs = 1.f, sn = 0.f;
    if (ok) {
      const size_t row = (((size_t)b * p.L + t0 + t) * RG + r * p.G + g) * N;
      const float* bb = p.b_bias + ((size_t)h * p.R + r) * N;
      const float* cb = p.c_bias + ((size_t)h * p.R + r) * N;
      if (j < A) {
        sincos_acc(theta_at(p, bh, t0 + t, j), &sn, &cs);
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
    Kc[v * ns + n0] = k0;
    Qc[v * ns + n0] = q0;
    if (j < A) {
      Kc[v * ns + j + A] = k1;
      Qc[v * ns + j + A] = q1;
      if (cs_l) {
        cs_l[v * A + j] = cs;
        sn_l[v * A + j] = sn;
      }
    }
  }
  const int pad = p.NT * 16 - N;
  for (int it = tid; it < BQ * pad; it += nthr) {
    const int v = it / pad, n = N + (it - v * pad);
    Kc[v * ns + n] = 0.f;
    Qc[v * ns + n] = 0.f;
  }
}

// X_v = x_t * mimo_x[h, r] of the chunk's virtual rows into LDS (stride ps),
// times wx[t] when wx is given; with xt also the raw x rows [Qt][ps].
__device__ void load_x_m(const BwdK& p, int b, int h, int t0, int nv, float* X, int ps, const float* wx,
                         float* xt, int tid, int nthr) {
  const int P = p.P, PP = p.PT * 16;
  for (int it = tid; it < BQ * PP; it += nthr) {
    const int v = it / PP, pp = it - v * PP;
    const int t = v >> p.rsl, r = v & (p.RS - 1);
    float xv = 0.f;
    if (t < nv && r < p.R && pp < P) {
      const float xr = p.x[(((size_t)b * p.L + t0 + t) * p.H + h) * P + pp];
      xv = xr * p.mimo_x[((size_t)h * p.R + r) * P + pp];
      if (xt && r == 0) xt[t * ps + pp] = xr;
      if (wx) xv *= wx[t];
    } else if (xt && r == 0 && t < p.Qt) {
      xt[t * ps + pp] = 0.f;
    }
    X[v * ps + pp] = xv;
  }
}

// load_kq_m with 16-byte accesses (conditions of load_kq4): item (virtual
// row v = t RS + r, four columns); rows of padding ranks or past the end are zero.
__device__ __forceinline__ void load_kq4_m(const BwdK& p, const Geom gm, int b, int h, int g, int t0, int nv,
                                           float* Kc, float* Qc, int ns, float* cs_l, float* sn_l, int tid) {
  const int N = gm.N, A = gm.A, A4 = A / 4, NP4 = (N - 2 * A) / 4;
  const int bh = b * p.H + h, R = p.R, G = p.G, RGN = R * G * N, rsl = p.rsl, rmask = p.RS - 1;
  const size_t row0 = ((size_t)b * p.L + t0) * RGN + (size_t)g * N;  // (t, r) at row0 + t R G N + r G N
  const float* bbh = p.b_bias + (size_t)h * R * N;                    // rank r at + r N
  const float* cbh = p.c_bias + (size_t)h * R * N;
  if (A > 0) {
    const float* th = p.theta + ((size_t)bh * p.L + t0) * A;
    const float* tp = p.tpre + ((size_t)bh * p.nT + t0 / TT) * A;  // a chunk lies inside one tile
    for (int it = tid; it < BQ * A4; it += 512) {
      const int v = it / A4, j = 4 * (it - v * A4);
      const int t = v >> rsl, r = v & rmask;
      const bool ok = t < nv && r < R;
      const int tc = min(t, nv - 1), rc = min(r, R - 1);
      const int ro = tc * RGN + rc * G * N, bo = rc * N;
      const floatx4 th4 = ldg4(th + tc * A + j), tp4 = ldg4(tp + j);
      const floatx4 b0 = ldg4(p.b + row0 + ro + j), b1 = ldg4(p.b + row0 + ro + j + A);
      const floatx4 c0 = ldg4(p.c + row0 + ro + j), c1 = ldg4(p.c + row0 + ro + j + A);
      const floatx4 bb0 = ldg4(bbh + bo + j), bb1 = ldg4(bbh + bo + j + A);
      const floatx4 cb0 = ldg4(cbh + bo + j), cb1 = ldg4(cbh + bo + j + A);
      floatx4 k0, k1, q0, q1, cs4, sn4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float sn, cs;
        sincos_acc(th4[e] + tp4[e], &sn, &cs);
        const float kb0 = b0[e] + bb0[e], kb1 = b1[e] + bb1[e];
        const float qc0 = c0[e] + cb0[e], qc1 = c1[e] + cb1[e];
        k0[e] = ok ? kb0 * cs - kb1 * sn : 0.f;
        k1[e] = ok ? kb0 * sn + kb1 * cs : 0.f;
        q0[e] = ok ? qc0 * cs - qc1 * sn : 0.f;
        q1[e] = ok ? qc0 * sn + qc1 * cs : 0.f;
        cs4[e] = cs;
        sn4[e] = sn;
      }
      sts4(Kc + v * ns + j, k0);
      sts4(Kc + v * ns + j + A, k1);
      sts4(Qc + v * ns + j, q0);
      sts4(Qc + v * ns + j + A, q1);
      if (cs_l) {
        sts4(cs_l + v * A + j, cs4);
        sts4(sn_l + v * A + j, sn4);
      }
    }
  }
  for (int it = tid; it < BQ * NP4; it += 512) {
    const int v = it / NP4, n = 2 * A + 4 * (it - v * NP4);
    const int t = v >> rsl, r = v & rmask;
    const bool ok = t < nv && r < R;
    const int tc = min(t, nv - 1), rc = min(r, R - 1);
    const int ro = tc * RGN + rc * G * N, bo = rc * N;
    const floatx4 b4 = ldg4(p.b + row0 + ro + n), c4 = ldg4(p.c + row0 + ro + n);
    const floatx4 bb4 = ldg4(bbh + bo + n), cb4 = ldg4(cbh + bo + n);
    floatx4 kv, qv;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kv[e] = ok ? b4[e] + bb4[e] : 0.f;
      qv[e] = ok ? c4[e] + cb4[e] : 0.f;
    }
    sts4(Kc + v * ns + n, kv);
    sts4(Qc + v * ns + n, qv);
  }
}

// load_x_m with 16-byte accesses (P a multiple of 16, 16-byte aligned rows):
// X_v = x_t mimo_x[h, r] (times wx[t]); with xt the raw x rows [Qt][ps].
__device__ __forceinline__ void load_x4_m(const BwdK& p, const Geom gm, int b, int h, int t0, int nv, float* X,
                                          int ps, const float* wx, float* xt, int tid) {
  const int P = gm.P, P4 = P / 4, HP = p.H * P, R = p.R, rsl = p.rsl, rmask = p.RS - 1;
  const size_t row0 = (((size_t)b * p.L + t0) * p.H + h) * P;
  const float* mx = p.mimo_x + (size_t)h * R * P;
  for (int it = tid; it < BQ * P4; it += 512) {
    const int v = it / P4, pp = 4 * (it - v * P4);
    const int t = v >> rsl, r = v & rmask;
    const bool ok = t < nv && r < R;
    const floatx4 x4 = ldg4(p.x + row0 + min(t, nv - 1) * HP + pp);
    const floatx4 w4 = ldg4(mx + min(r, R - 1) * P + pp);
    const float sx = wx ? wx[t] : 1.f;
    floatx4 xv, xr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xv[e] = ok ? x4[e] * w4[e] * sx : 0.f;
      xr[e] = t < nv ? x4[e] : 0.f;
    }
    sts4(X + v * ps + pp, xv);
    if (xt && r == 0) sts4(xt + t * ps + pp, xr);
  }
}

// Mask weights between virtual rows: M[v][w] and V[v][w] as for tokens, by
// the tokens of the rows.
__device__ __forceinline__ void row_masks(int tv, int tw, const float* cum, const float* scl, const float* gam,
                                          float* m, float* dec) {
  *dec = tw < tv ? expf(cum[tv] - cum[tw]) : 0.f;
  *m = tw < tv ? *dec * scl[tw] : (tw == tv ? gam[tv] : 0.f);
}

// (M2) Per chunk: forward summary S = sum_v e^(cumx-cum_t) s_t X_v K_v^T and the decay.
// NC > 0: geometry fixed at (NC, PC, AC) with the 16-byte loaders.
template <int NC, int PC, int AC>
__global__ __launch_bounds__(512) void mimo_summary_kernel(BwdK p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const Geom gm = geom_of<NC, PC, AC>(p);
  const int NS = gm.NT * 16 + 4, PS = gm.PT * 16 + 4, P = gm.P, N = gm.N;
  float* Kc = lds;
  float* Qc = Kc + BQ * NS;  // loaded with the keys; unused here
  float* Xw = Qc + BQ * NS;
  float* cum = Xw + BQ * PS;
  float* scl = cum + BQ;
  float* gam = scl + BQ;
  float* ec = gam + BQ;
  float* ex = ec + BQ;
  float* wx = ex + BQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int bh = blockIdx.x / p.nc, c = blockIdx.x - bh * p.nc;
  const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
  const int t0 = c * p.Qt, nv = min(p.Qt, p.L - t0);
  if (wave == 0) chunk_scalars(p, b, h, t0, nv, ChunkScalars{cum, scl, gam, ec, ex}, lane);
  if constexpr (NC > 0)
    load_kq4_m(p, gm, b, h, g, t0, nv, Kc, Qc, NS, nullptr, nullptr, tid);
  else
    load_kq_m(p, b, h, g, t0, nv, Kc, Qc, NS, nullptr, nullptr, tid, blockDim.x);
  __syncthreads();
  if (tid < BQ) wx[tid] = ex[tid] * scl[tid];
  __syncthreads();
  if constexpr (NC > 0)
    load_x4_m(p, gm, b, h, t0, nv, Xw, PS, wx, nullptr, tid);
  else
    load_x_m(p, b, h, t0, nv, Xw, PS, wx, nullptr, tid, blockDim.x);
  __syncthreads();
  if (tid == 0) p.decay[blockIdx.x] = expf(cum[BQ - 1]);
  const int ntile = gm.PT * gm.NT;
  float* dst = p.hs + (size_t)blockIdx.x * P * N;
  const int r = lane & 15, q = lane >> 4;
  for (int job = wave; job < ntile; job += nw) {
    const int pt = job / gm.NT, nt = job - pt * gm.NT;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mm_tile(Xw + pt * 16, 1, PS, Kc + nt * 16, NS, 1, BQ, acc, lane);
    const int n = nt * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pp = pt * 16 + 4 * q + i;
      if (pp < P && n < N) dst[pp * N + n] = acc[i];
    }
  }
}

constexpr float kMimoNormEpsBwd = 1.0e-5f;  // the MIMO output-norm epsilon of the MIMO push constants

// Sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_sum(float v) { return read_lane_f(scan64_f(v), 63); }

// (M4) Per chunk: the per-rank read-outs y_v = e^cum_t Q_v h'_e^T + (M o Q K^T) X,
// then the MIMO epilogue's adjoint per token (mimo_o, output norm, gate, D):
// gy_v (stored), d_z, rho_t and per-chunk partial sums of the weight
// gradients; last the reverse summary sum_v e^cum_t gy_v Q_v^T.  The
// per-rank weights and the chunk's dout / z rows are staged in LDS with the
// other operands, so the epilogue loop waits on no memory.
template <bool VEC4, int RSC, int NC, int PC, int AC>
__global__ __launch_bounds__(512, 4) void mimo_post_kernel(BwdK p) {
  constexpr bool FIX = NC > 0;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const Geom gm = geom_of<NC, PC, AC>(p);
  const int NS = gm.NT * 16 + 4, PS = gm.PT * 16 + 4, PP = gm.PT * 16, NN = gm.NT * 16;
  float* Kc = lds;
  float* Qc = Kc + BQ * NS;
  float* X = Qc + BQ * NS;
  float* Y = X + BQ * PS;
  float* GY = Y + BQ * PS;
  float* MQK = GY + BQ * PS;
  float* red = MQK + BQ * MS;        // [8][RS P] cross-wave partials
  float* WZ = red + 8 * p.RS * PP;   // mimo_z [R][P]
  float* WO = WZ + p.R * gm.P;       // mimo_o [R][P]
  float* WN = WO + p.R * gm.P;       // norm_weight [P]
  float* GO = WN + gm.P;             // dout of the chunk's tokens [Qt][P]
  float* ZT = GO + p.Qt * gm.P;      // z of the chunk's tokens [Qt][P]
  float* cum = ZT + p.Qt * gm.P;
  float* scl = cum + BQ;
  float* gam = scl + BQ;
  float* ec = gam + BQ;
  float* ex = ec + BQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int bh = blockIdx.x / p.nc, c = blockIdx.x - bh * p.nc;
  const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
  const int t0 = c * p.Qt, nv = min(p.Qt, p.L - t0);
  const int P = gm.P, N = gm.N, H = p.H, R = p.R, rsl = p.rsl;
  const float* HEg = p.hs + (size_t)blockIdx.x * P * N;
  if (wave == 0) chunk_scalars(p, b, h, t0, nv, ChunkScalars{cum, scl, gam, ec, ex}, lane);
  if constexpr (FIX) {
    load_kq4_m(p, gm, b, h, g, t0, nv, Kc, Qc, NS, nullptr, nullptr, tid);
    load_x4_m(p, gm, b, h, t0, nv, X, PS, nullptr, nullptr, tid);
  } else {
    load_kq_m(p, b, h, g, t0, nv, Kc, Qc, NS, nullptr, nullptr, tid, blockDim.x);
    load_x_m(p, b, h, t0, nv, X, PS, nullptr, nullptr, tid, blockDim.x);
  }
  for (int i = tid; i < R * P; i += blockDim.x) {
    WZ[i] = p.has_z ? p.mimo_z[(size_t)h * R * P + i] : 0.f;
    WO[i] = p.mimo_o[(size_t)h * R * P + i];
  }
  for (int i = tid; i < P; i += blockDim.x) WN[i] = p.has_norm ? p.norm_weight[(size_t)h * P + i] : 0.f;
  for (int i = tid; i < p.Qt * P; i += blockDim.x) {
    const int t = i / P, pp = i - t * P;
    const size_t gi = (((size_t)b * p.L + t0 + min(t, nv - 1)) * H + h) * P + pp;
    GO[i] = t < nv ? p.dout[gi] : 0.f;
    ZT[i] = (t < nv && p.has_z) ? p.z[gi] : 0.f;
  }
  __syncthreads();
  const int r = lane & 15, q = lane >> 4;
  if (wave < 4) {  // masked Q K^T
    const int mt = wave >> 1, st = wave & 1;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mm_tile_k4(Qc + mt * 16 * NS, NS, Kc + st * 16 * NS, NS, NN, acc, lane);
    const int w = st * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = mt * 16 + 4 * q + i;
      const int tv = v >> rsl, tw = w >> rsl;
      float m, dec;
      if constexpr (FIX) {
        dec = tw < tv ? exp_fast(cum[tv] - cum[tw]) : 0.f;
        m = tw < tv ? dec * scl[tw] : (tw == tv ? gam[tv] : 0.f);
      } else {
        row_masks(tv, tw, cum, scl, gam, &m, &dec);
      }
      MQK[v * MS + w] = m * acc[i];
    }
  }
  __syncthreads();
  if constexpr (FIX) {
    // y tiles: waves w and w + 4 share head_dim tile w (PT == 4), each over
    // one half of the state columns and both row halves, so each state tile
    // is read from global memory once; they swap partial products through
    // the key rows (dead after the masked Q K^T) and wave w + 4 h finishes
    // row half h, summing the state halves in order.
    static_assert(PC == 64, "four head_dim tiles, two waves each");
    const int pt = wave & 3, kh = wave >> 2;
    const float* Sg = HEg + (pt * 16 + r) * N + (NC / 2) * kh + 4 * q;
    floatx4 sv[NC / 32];
#pragma unroll
    for (int j = 0; j < NC / 32; ++j) sv[j] = ldg4(Sg + 16 * j);
    floatx4 part[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      floatx4 a1 = {0.f, 0.f, 0.f, 0.f};
      const float* ap = Qc + (mt * 16 + r) * NS + (NC / 2) * kh + 4 * q;
#pragma unroll
      for (int j = 0; j < NC / 32; ++j) {
        const floatx4 av = lds_read4(ap + 16 * j);
        a1 = mfma16(av[0], sv[j][0], a1);
        a1 = mfma16(av[1], sv[j][1], a1);
        a1 = mfma16(av[2], sv[j][2], a1);
        a1 = mfma16(av[3], sv[j][3], a1);
      }
      part[mt] = a1;
    }
    float* xch = Kc;  // [8 waves][64 lanes] float4
    sts4(xch + (wave * 64 + lane) * 4, kh ? part[0] : part[1]);
    __syncthreads();
    const floatx4 other = lds_read4(xch + ((wave ^ 4) * 64 + lane) * 4);
    const int mt = kh;
    const floatx4 a1 = kh ? other + part[1] : part[0] + other;
    floatx4 a2 = {0.f, 0.f, 0.f, 0.f};
    a2 = mm_tile(MQK + mt * 16 * MS, MS, 1, X + pt * 16, PS, 1, BQ, a2, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = mt * 16 + 4 * q + i;
      Y[v * PS + pt * 16 + r] = fmaf(ec[v >> rsl], a1[i], a2[i]);
    }
  } else {
    for (int job = wave; job < 2 * gm.PT; job += nw) {  // y tiles
      const int mt = job / gm.PT, pt = job - mt * gm.PT;
      floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
      if constexpr (VEC4)
        a1 = mm_tile_k4_g<8>(Qc + mt * 16 * NS, NS, HEg + (size_t)pt * 16 * N, N, P - pt * 16, N, NN, a1, lane);
      else
        a1 = mm_tile_k1_g<32>(Qc + mt * 16 * NS, NS, HEg + (size_t)pt * 16 * N, N, P - pt * 16, N, NN, a1, lane);
      a2 = mm_tile(MQK + mt * 16 * MS, MS, 1, X + pt * 16, PS, 1, BQ, a2, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = mt * 16 + 4 * q + i;
        Y[v * PS + pt * 16 + r] = fmaf(ec[v >> rsl], a1[i], a2[i]);
      }
    }
  }
  __syncthreads();

  // epilogue adjoint: wave w owns tokens w, w + 8, ...; lanes over head_dim (two per lane)
  const float Dh = p.has_d ? p.d[h] : 0.f;
  float mo_acc[RSC][2], mz_acc[RSC][2], nw_acc[2] = {0.f, 0.f}, dd_acc = 0.f;
#pragma unroll
  for (int rr = 0; rr < RSC; ++rr) mo_acc[rr][0] = mo_acc[rr][1] = mz_acc[rr][0] = mz_acc[rr][1] = 0.f;
  for (int t = wave; t < p.Qt; t += nw) {
    const bool tok = t < nv;
    const size_t ti = (((size_t)b * p.L + t0 + min(t, nv - 1)) * H + h) * P;
    float go[2], zv[2], dz[2] = {0.f, 0.f}, rho = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pp = lane + 64 * k;
      go[k] = pp < P ? GO[t * P + pp] : 0.f;
      zv[k] = pp < P ? ZT[t * P + pp] : 0.f;
    }
#pragma unroll
    for (int rr = 0; rr < RSC; ++rr) {
      const int v = (t << rsl) + rr;
      const bool ok = tok && rr < R;
      float y2[2], y3[2], sil[2], u[2], y1v[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pp = lane + 64 * k;
        const bool in = ok && pp < P;
        y1v[k] = in ? Y[v * PS + pp] : 0.f;
        y2[k] = fmaf(Dh, in ? X[v * PS + pp] : 0.f, y1v[k]);
        const float mz = in ? WZ[rr * P + pp] : 0.f;
        u[k] = zv[k] * mz;
        sil[k] = p.has_z ? (FIX ? sigmoid_fast(u[k]) * u[k] : siluf_acc(u[k])) : 1.f;
        y3[k] = y2[k] * sil[k];
      }
      float rinv = 1.f, yn[2] = {y3[0], y3[1]}, nwv[2] = {1.f, 1.f};
      if (p.has_norm) {
        const float ss = wave_sum(y3[0] * y3[0] + y3[1] * y3[1]);
        rinv = 1.f / sqrtf(ss / (float)P + kMimoNormEpsBwd);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int pp = lane + 64 * k;
          yn[k] = y3[k] * rinv;
          nwv[k] = (ok && pp < P) ? WN[pp] : 0.f;
        }
      }
      float g4[2], g3[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pp = lane + 64 * k;
        const float mo = (ok && pp < P) ? WO[rr * P + pp] : 0.f;
        const float y4 = p.has_norm ? yn[k] * nwv[k] : y3[k];
        mo_acc[rr][k] = fmaf(go[k], y4, mo_acc[rr][k]);
        g4[k] = go[k] * mo;
      }
      if (p.has_norm) {
        float gn[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          nw_acc[k] = fmaf(g4[k], yn[k], nw_acc[k]);
          gn[k] = g4[k] * nwv[k];
        }
        const float mg = wave_sum(gn[0] * yn[0] + gn[1] * yn[1]) / (float)P;
#pragma unroll
        for (int k = 0; k < 2; ++k) g3[k] = rinv * (gn[k] - yn[k] * mg);
      } else {
        g3[0] = g4[0];
        g3[1] = g4[1];
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pp = lane + 64 * k;
        float g2 = g3[k];
        if (p.has_z) {
          const float du = g3[k] * y2[k] * (FIX ? dsilu_fast(u[k]) : dsilu_acc(u[k]));
          const float mz = (ok && pp < P) ? WZ[rr * P + pp] : 0.f;
          mz_acc[rr][k] = fmaf(du, zv[k], mz_acc[rr][k]);
          dz[k] = fmaf(du, mz, dz[k]);
          g2 = g3[k] * sil[k];
        }
        if (!(ok && pp < P)) g2 = 0.f;
        rho = fmaf(g2, y1v[k], rho);
        dd_acc = fmaf(g2, (ok && pp < P) ? X[v * PS + pp] : 0.f, dd_acc);
        if (pp < PP) GY[v * PS + pp] = g2;
        if (pp < P) p.gyr[((size_t)blockIdx.x * BQ + v) * P + pp] = g2;
      }
    }
    if (tok) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pp = lane + 64 * k;
        if (pp < P) p.d_z[ti + pp] = dz[k];
      }
      const float rs = wave_sum(rho);
      if (lane == 0) p.rho[(size_t)bh * p.L + t0 + t] = rs;
    }
  }
  // per-chunk partial sums of the weight gradients: waves in order
  const int RP = p.RS * PP;
  const size_t cp = (size_t)blockIdx.x;
  for (int which = 0; which < 3; ++which) {
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RSC; ++rr) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pp = lane + 64 * k;
        if (pp < PP) {
          const float v = which == 0 ? mo_acc[rr][k] : which == 1 ? mz_acc[rr][k] : (rr == 0 ? nw_acc[k] : 0.f);
          red[wave * RP + rr * PP + pp] = v;
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < (which == 2 ? P : R * P); i += blockDim.x) {
      const int rr = i / P, pp = i - rr * P;
      float s = 0.f;
      for (int w = 0; w < nw; ++w) s += red[w * RP + rr * PP + pp];
      if (which == 0) p.mo_part[cp * R * P + i] = s;
      else if (which == 1) p.mz_part[cp * R * P + i] = s;
      else p.nw_part[cp * P + i] = s;
    }
  }
  {
    const float dsum = wave_sum(dd_acc);
    __syncthreads();
    if (lane == 0) red[wave] = dsum;
    __syncthreads();
    if (tid == 0) {
      float s = 0.f;
      for (int w = 0; w < nw; ++w) s += red[w];
      p.dd_part[cp] = s;
    }
  }
  // reverse summary: [p][n] = sum_v e^cum_t gy_v[p] Q_v[n]
  __syncthreads();
  for (int it = tid; it < BQ * PP; it += blockDim.x) {
    const int v = it / PP, pp = it - v * PP;
    Y[v * PS + pp] = ec[v >> rsl] * GY[v * PS + pp];
  }
  __syncthreads();
  const size_t base = (size_t)blockIdx.x * P * N;
  for (int job = wave; job < gm.PT * gm.NT; job += nw) {
    const int pt = job / gm.NT, nt = job - pt * gm.NT;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = mm_tile(Y + pt * 16, 1, PS, Qc + nt * 16, NS, 1, BQ, acc, lane);
    const int n = nt * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pp = pt * 16 + 4 * q + i;
      if (pp < P && n < N) p.gs[base + (size_t)pp * N + n] = acc[i];
    }
  }
}

struct MimoChunkLds {
  int NS, PS;
  int o_kc, o_qc, o_x, o_gy, o_dx, o_xt, o_vv, o_msg, o_sqd, o_sgd, o_cs, o_sn, o_sc, o_part, total;
};

__host__ __device__ inline MimoChunkLds mimo_chunk_lds(int PT, int NT, int A, int RS, int Qt) {
  MimoChunkLds l{};
  l.NS = NT * 16 + 4;
  l.PS = PT * 16 + 4;
  int off = 0;
  l.o_kc = off; off += BQ * l.NS;
  l.o_qc = off; off += BQ * l.NS;
  l.o_x = off;
  l.o_gy = off + BQ * l.PS;
  off += 2 * BQ * l.PS > BQ * l.NS ? 2 * BQ * l.PS : BQ * l.NS;  // x, gy; then the dQ / dK staging
  l.o_dx = off; off += BQ * l.PS;                                // dX_v
  l.o_xt = off; off += Qt * l.PS;                                // raw x per token
  l.o_vv = off; off += BQ * MS;
  l.o_msg = off; off += BQ * MS;                                 // then d theta [Qt][A]
  l.o_sqd = off; off += BQ * RS;                                 // same-token Q_v . K_w
  l.o_sgd = off; off += BQ * RS;                                 // same-token gy_v . X_w
  l.o_cs = off; off += BQ * A;
  l.o_sn = off; off += BQ * A;
  l.o_sc = off; off += 5 * BQ;
  l.o_part = off; off += BQ * PT;                                // ds partials
  l.total = off;
  return l;
}

// (M6) Per chunk: G K, dQ, dK of the virtual rows on FP32 MFMA with gy from
// the post kernel; d x (rank sum of mimo_x dX_r), partial mimo_x sums, the
// per-head rank-row adjoints of B + b_bias and C + c_bias, and the local
// suffix sums of the d adt terms and of d theta.  NC > 0: geometry fixed at
// (NC, PC, AC) as for bwd_chunk_kernel.
template <bool VEC4, int NC, int PC, int AC>
__global__ __launch_bounds__(512, 4) void mimo_chunk_kernel(BwdK p) {
  constexpr bool FIX = NC > 0;
  static_assert(!FIX || (NC == 128 && PC % 16 == 0 && AC % 4 == 0 && (BQ * AC / 4) % 64 == 0),
                "fixed geometry: N = 128 (one state tile per wave), P a multiple of 16");
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const Geom gm = geom_of<NC, PC, AC>(p);
  const MimoChunkLds ll = mimo_chunk_lds(gm.PT, gm.NT, gm.A, p.RS, p.Qt);
  const int NS = ll.NS, PS = ll.PS, PP = gm.PT * 16, NN = gm.NT * 16;
  float* Kc = lds + ll.o_kc;
  float* Qc = lds + ll.o_qc;
  float* X = lds + ll.o_x;
  float* GY = lds + ll.o_gy;
  float* DX = lds + ll.o_dx;
  float* XT = lds + ll.o_xt;
  float* VV = lds + ll.o_vv;
  float* MSG = lds + ll.o_msg;
  float* SQD = lds + ll.o_sqd;
  float* SGD = lds + ll.o_sgd;
  float* CS = lds + ll.o_cs;
  float* SN = lds + ll.o_sn;
  float* cum = lds + ll.o_sc;
  float* scl = cum + BQ;
  float* gam = scl + BQ;
  float* ec = gam + BQ;
  float* ex = ec + BQ;
  float* ds_part = lds + ll.o_part;  // [BQ][PT]
  float* STG = X;                    // after the products: dQ, then dK [BQ][NS]
  float* DTH = MSG;                  // after the products: d theta [Qt][A]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / p.nc, c = blockIdx.x - bh * p.nc;
  const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
  const int t0 = c * p.Qt, nv = min(p.Qt, p.L - t0);
  const int P = gm.P, N = gm.N, H = p.H, A = gm.A, NP = N - A, R = p.R, RS = p.RS, rsl = p.rsl;
  const float* HEg = p.hs + (size_t)blockIdx.x * P * N;
  const float* GXg = p.gs + (size_t)blockIdx.x * P * N;
  const float* gyc = p.gyr + (size_t)blockIdx.x * BQ * P;  // row v at gyc + v P

  if (wave == 0) chunk_scalars(p, b, h, t0, nv, ChunkScalars{cum, scl, gam, ec, ex}, lane);
  if constexpr (FIX) {
    load_kq4_m(p, gm, b, h, g, t0, nv, Kc, Qc, NS, CS, SN, tid);
    load_x4_m(p, gm, b, h, t0, nv, X, PS, nullptr, XT, tid);
    constexpr int P4 = PC / 4;
    for (int it = tid; it < BQ * P4; it += 512) {
      const int v = it / P4, pp = 4 * (it - v * P4);
      sts4(GY + v * PS + pp, ldg4(gyc + v * P + pp));
    }
  } else {
    load_kq_m(p, b, h, g, t0, nv, Kc, Qc, NS, CS, SN, tid, 512);
    load_x_m(p, b, h, t0, nv, X, PS, nullptr, XT, tid, 512);
    for (int it = tid; it < BQ * PP; it += 512) {
      const int v = it / PP, pp = it - v * PP;
      GY[v * PS + pp] = pp < P ? gyc[v * P + pp] : 0.f;
    }
  }
  __syncthreads();
  const float Dh = p.has_d ? p.d[h] : 0.f;
  const int r = lane & 15, q = lane >> 4;

  // masked Q K^T (waves 0-3) and gy X^T (waves 4-7), and their same-token blocks
  {
    const bool sgx = wave >= 4;
    const int mt = (wave & 3) >> 1, st = wave & 1;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    if (!sgx)
      acc = mm_tile_k4(Qc + mt * 16 * NS, NS, Kc + st * 16 * NS, NS, NN, acc, lane);
    else
      acc = mm_tile_k4(GY + mt * 16 * PS, PS, X + st * 16 * PS, PS, PP, acc, lane);
    const int w = st * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = mt * 16 + 4 * q + i;
      const int tv = v >> rsl, tw = w >> rsl;
      float m, dec;
      if constexpr (FIX) {
        dec = tw < tv ? exp_fast(cum[tv] - cum[tw]) : 0.f;
        m = tw < tv ? dec * scl[tw] : (tw == tv ? gam[tv] : 0.f);
      } else {
        row_masks(tv, tw, cum, scl, gam, &m, &dec);
      }
      if (!sgx) {
        VV[v * MS + w] = dec * acc[i];
        if (tv == tw) SQD[v * RS + (w & (RS - 1))] = acc[i];
      } else {
        MSG[v * MS + w] = m * acc[i];
        if (tv == tw) SGD[v * RS + (w & (RS - 1))] = acc[i];
      }
    }
  }
  __syncthreads();

  // G K tiles: dX_v = D gy_v + s_t G K_v + lam_t dt_t sum_{w in t} (Q_w . K_v) gy_w
  const int nY = 2 * gm.PT, nQ = 2 * gm.NT;
  for (int job = wave; job < nY; job += 8) {
    const int mt = job / gm.PT, pt = job - mt * gm.PT;
    floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
    const float* Sg = GXg + (size_t)pt * 16 * N;
    if constexpr (VEC4)
      a1 = mm_tile_k4_g<8>(Kc + mt * 16 * NS, NS, Sg, N, P - pt * 16, N, NN, a1, lane);
    else
      a1 = mm_tile_k1_g<32>(Kc + mt * 16 * NS, NS, Sg, N, P - pt * 16, N, NN, a1, lane);
    a2 = mm_tile(VV + mt * 16, 1, MS, GY + pt * 16, PS, 1, BQ, a2, lane);
    const int pp = pt * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = mt * 16 + 4 * q + i;
      const int tv = v >> rsl, rv = v & (RS - 1);
      const float gk = fmaf(ex[tv], a1[i], a2[i]);
      float same = 0.f;
      for (int rw = 0; rw < RS; ++rw) {
        const int w = (tv << rsl) + rw;
        same = fmaf(SQD[w * RS + rv], GY[w * PS + pp], same);
      }
      DX[v * PS + pp] = fmaf(Dh, GY[v * PS + pp], fmaf(scl[tv], gk, gam[tv] * same));
      const bool ok = tv < nv && rv < R && pp < P;
      const float part = row16_sum(ok ? X[v * PS + pp] * gk : 0.f);
      if (r == 15) ds_part[v * gm.PT + pt] = part;
    }
  }
  floatx4 res[4];
  if constexpr (FIX) {
    // as in bwd_chunk_kernel: wave w owns state columns 16 w .. 16 w + 15
    const int nt = wave;
    float sh[PC / 4], sg[PC / 4];
#pragma unroll
    for (int j = 0; j < PC / 4; ++j) {
      sh[j] = HEg[(4 * j + q) * N + nt * 16 + r];
      sg[j] = GXg[(4 * j + q) * N + nt * 16 + r];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool isdk = k >= 2;
      const int mt = k & 1;
      floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
      const float* Ar = (isdk ? X : GY) + (mt * 16 + r) * PS + q;
#pragma unroll
      for (int j = 0; j < PC / 4; ++j) a1 = mfma16(Ar[4 * j], isdk ? sg[j] : sh[j], a1);
      if (!isdk)
        a2 = mm_tile(MSG + mt * 16 * MS, MS, 1, Kc + nt * 16, NS, 1, BQ, a2, lane);
      else
        a2 = mm_tile(MSG + mt * 16, 1, MS, Qc + nt * 16, NS, 1, BQ, a2, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tv = (mt * 16 + 4 * q + i) >> rsl;
        const float wgt = isdk ? scl[tv] * ex[tv] : ec[tv];
        res[k][i] = fmaf(wgt, a1[i], a2[i]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int job = wave + 8 * k;
      res[k] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (job < 2 * nQ) {
        const bool isdk = job >= nQ;
        const int jj = isdk ? job - nQ : job;
        const int mt = jj / gm.NT, nt = jj - mt * gm.NT;
        floatx4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
        const float* Sg = (isdk ? GXg : HEg) + nt * 16;
        if (!isdk) {
          a1 = mm_tile_g<32>(GY + mt * 16 * PS, PS, Sg, N, P, N - nt * 16, PP, a1, lane);
          a2 = mm_tile(MSG + mt * 16 * MS, MS, 1, Kc + nt * 16, NS, 1, BQ, a2, lane);
        } else {
          a1 = mm_tile_g<32>(X + mt * 16 * PS, PS, Sg, N, P, N - nt * 16, PP, a1, lane);
          a2 = mm_tile(MSG + mt * 16, 1, MS, Qc + nt * 16, NS, 1, BQ, a2, lane);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tv = (mt * 16 + 4 * q + i) >> rsl;
          const float wgt = isdk ? scl[tv] * ex[tv] : ec[tv];
          res[k][i] = fmaf(wgt, a1[i], a2[i]);
        }
      }
    }
  }
  __syncthreads();  // DX complete; x, gy, the masks free after this point

  // d x = sum_r mimo_x[h, r] dX_r, and per-chunk partial sums of dX_r * x for d mimo_x
  const size_t xrow0 = (((size_t)b * p.L + t0) * H + h) * P;  // token t at xrow0 + t H P
  const float* mxh = p.mimo_x + (size_t)h * R * P;
  for (int it = tid; it < p.Qt * P; it += 512) {
    const int t = it / P, pp = it - t * P;
    if (t < nv) {
      float s = 0.f;
      for (int rr = 0; rr < R; ++rr) s = fmaf(mxh[rr * P + pp], DX[((t << rsl) + rr) * PS + pp], s);
      p.d_x[xrow0 + t * H * P + pp] = s;
    }
  }
  for (int it = tid; it < R * P; it += 512) {
    const int rr = it / P, pp = it - rr * P;
    float s = 0.f;
    for (int t = 0; t < nv; ++t) s = fmaf(DX[((t << rsl) + rr) * PS + pp], XT[t * PS + pp], s);
    p.mx_part[(size_t)blockIdx.x * R * P + it] = s;
  }

  // the per-token sums before the masks' region is reused for d theta
  float e_tok = 0.f, ds_tok = 0.f;
  if (wave == 0 && lane < nv) {
    for (int rr = 0; rr < R; ++rr) {
      const int v = (lane << rsl) + rr;
      for (int pt = 0; pt < gm.PT; ++pt) ds_tok += ds_part[v * gm.PT + pt];
      for (int rw = 0; rw < R; ++rw) {
        const int w = (lane << rsl) + rw;
        e_tok = fmaf(SGD[w * RS + rr], SQD[w * RS + rr], e_tok);
      }
    }
    e_tok += ds_tok;
  }

  // rotation adjoints: queries, then keys, staged through LDS
  const size_t hrow0 = (((size_t)b * p.L + t0) * H + h) * R * N;  // (t, r) at hrow0 + (t H R + r) N
  const int HRN = H * R * N;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int job = wave + 8 * k;
      if (job < 2 * nQ && (job >= nQ) == (pass == 1)) {
        const int jj = pass ? job - nQ : job;
        const int mt = jj / gm.NT, nt = jj - mt * gm.NT;
#pragma unroll
        for (int i = 0; i < 4; ++i) STG[(mt * 16 + 4 * q + i) * NS + nt * 16 + r] = res[k][i];
      }
    }
    __syncthreads();
    const float* Rw = pass ? Kc : Qc;
    float* dst = (pass ? p.db_head : p.dc_head) + hrow0;
    if constexpr (FIX) {
      constexpr int A4 = AC / 4, NP4 = (NC - 2 * AC) / 4;
      // rotated columns: item (token, four angles), ranks summed into d theta
      for (int it = tid; it < p.Qt * A4; it += 512) {
        const int t = it / A4, j = 4 * (it - t * A4);
        if (t >= nv) {
          if (pass == 0) sts4(DTH + t * A + j, floatx4{0.f, 0.f, 0.f, 0.f});
          continue;
        }
        floatx4 dth = pass ? lds_read4(DTH + t * A + j) : floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int rr = 0; rr < R; ++rr) {
          const int v = (t << rsl) + rr;
          const floatx4 cs = lds_read4(CS + v * A + j), sn = lds_read4(SN + v * A + j);
          const floatx4 d0 = lds_read4(STG + v * NS + j), d1 = lds_read4(STG + v * NS + j + A);
          const floatx4 r0 = lds_read4(Rw + v * NS + j), r1 = lds_read4(Rw + v * NS + j + A);
          floatx4 u0, u1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[e] += d1[e] * r0[e] - d0[e] * r1[e];
            u0[e] = d0[e] * cs[e] + d1[e] * sn[e];
            u1[e] = d1[e] * cs[e] - d0[e] * sn[e];
          }
          const int o = (t * H * R + rr) * N;
          sts4(dst + o + j, u0);
          sts4(dst + o + j + A, u1);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dth[e] = pass ? dth[e] + acc[e] : acc[e];
        sts4(DTH + t * A + j, dth);
      }
      // plain columns: item (virtual row, four columns)
      for (int it = tid; it < BQ * NP4; it += 512) {
        const int v = it / NP4, n = 2 * AC + 4 * (it - v * NP4);
        const int t = v >> rsl, rr = v & (RS - 1);
        if (t < nv && rr < R) sts4(dst + (t * H * R + rr) * N + n, lds_read4(STG + v * NS + n));
      }
    } else {
      for (int it = tid; it < p.Qt * NP; it += 512) {
        const int t = it / NP, j = it - t * NP;
        if (t >= nv) {
          if (j < A && pass == 0) DTH[t * A + j] = 0.f;
          continue;
        }
        float dth = 0.f;
        for (int rr = 0; rr < R; ++rr) {
          const int v = (t << rsl) + rr;
          const int o = (t * H * R + rr) * N;
          if (j < A) {
            const float cs = CS[v * A + j], sn = SN[v * A + j];
            const float d0 = STG[v * NS + j], d1 = STG[v * NS + j + A];
            dth += d1 * Rw[v * NS + j] - d0 * Rw[v * NS + j + A];
            dst[o + j] = d0 * cs + d1 * sn;
            dst[o + j + A] = d1 * cs - d0 * sn;
          } else {
            dst[o + j + A] = STG[v * NS + j + A];
          }
        }
        if (j < A) DTH[t * A + j] = pass ? DTH[t * A + j] + dth : dth;
      }
    }
  }
  __syncthreads();

  // chunk-local suffix sums over the tokens
  if (wave == 0) {
    float phi = 0.f;
    if (lane < nv) {
      const size_t ri = (size_t)bh * p.L + t0 + lane;
      phi = p.rho[ri] - (scl[lane] - gam[lane]) * ds_tok - gam[lane] * e_tok;
      p.dsv[ri] = ds_tok;
      p.ev[ri] = e_tok;
    }
    const float loc = suffix_sum<32>(lane < 32 ? phi : 0.f, lane);
    if (lane < nv) p.d_adt[((size_t)b * p.L + t0 + lane) * H + h] = loc;
    if (lane == 0) p.phi_tot[blockIdx.x] = loc;
  } else if (tid >= 64 && tid < 64 + A) {
    const int a = tid - 64;
    float s = 0.f;
    float* dstp = p.dtheta + ((size_t)bh * p.L + t0) * A + a;
    for (int t = nv - 1; t >= 0; --t) {
      s += DTH[t * A + a];
      dstp[t * A] = s;
    }
    p.th_tot[(size_t)blockIdx.x * A + a] = s;
  }
}

// (M10) mimo_x / mimo_z / mimo_o / norm_weight gradients: sums of the chunk
// partials over batch and chunks.  A workgroup of 16 waves takes 64
// consecutive columns of one head's [R P] (or [P]) block (lane = column),
// wave w the (batch, chunk) pairs w, w + 16, ... in order, and the 16 wave
// sums are added in order.
__global__ __launch_bounds__(1024) void mimo_weights_kernel(BwdK p) {
  __shared__ float red[16][64];
  const int RP = p.R * p.P, cb_rp = (RP + 63) / 64, cb_p = (p.P + 63) / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // workgroups: [which 0..2][h][cb_rp], then [h][cb_p] for the norm weight
  int blk = blockIdx.x, which, width;
  if (blk < 3 * p.H * cb_rp) {
    which = blk / (p.H * cb_rp);
    blk -= which * p.H * cb_rp;
    width = RP;
  } else {
    which = 3;
    blk -= 3 * p.H * cb_rp;
    width = p.P;
  }
  const int cbn = which == 3 ? cb_p : cb_rp;
  const int h = blk / cbn;
  const int col = (blk - h * cbn) * 64 + lane;
  const float* src = which == 0 ? p.mx_part : which == 1 ? p.mz_part : which == 2 ? p.mo_part : p.nw_part;
  float s = 0.f;
  if (col < width) {
    const int per = p.B * p.nc;
    for (int k = w; k < per; k += 16) {
      const int bb = k / p.nc, cc = k - bb * p.nc;
      s += src[(((size_t)bb * p.H + h) * p.nc + cc) * width + col];
    }
  }
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && col < width) {
    float t = red[0][lane];
    for (int k = 1; k < 16; ++k) t += red[k][lane];
    if (which == 0) p.d_mimo_x[(size_t)h * RP + col] = t;
    else if (which == 1) p.d_mimo_z[(size_t)h * RP + col] = p.has_z ? t : 0.f;
    else if (which == 2) p.d_mimo_o[(size_t)h * RP + col] = t;
    else p.d_norm_weight[(size_t)h * p.P + col] = p.has_norm ? t : 0.f;
  }
}

struct BwdLayout {
  size_t theta, tpre, hs, gs, decay, dtheta, dbh, dch, dsv, ev, phi, th, ddp, bias, total;
  int nc, nT, nrb;
};

BwdLayout bwd_layout(const ScanGeom& g) {
  BwdLayout w{};
  const size_t BH = (size_t)g.B * g.H;
  w.nc = (int)((g.L + BQ - 1) / BQ);
  w.nT = (int)((g.L + TT - 1) / TT);
  w.nrb = (int)(((size_t)g.B * g.L + RB - 1) / RB);
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += (n + 63) / 64 * 64;  // 256-byte aligned pieces
    return o;
  };
  w.theta = take(BH * g.L * g.A);
  w.tpre = take(BH * w.nT * g.A);
  w.hs = take(BH * w.nc * g.P * g.N);
  w.gs = take(BH * w.nc * g.P * g.N);
  w.decay = take(BH * w.nc);
  w.dtheta = take(BH * g.L * g.A);
  w.dbh = take((size_t)g.B * g.L * g.H * g.N);
  w.dch = take((size_t)g.B * g.L * g.H * g.N);
  w.dsv = take(BH * g.L);
  w.ev = take(BH * g.L);
  w.phi = take(BH * w.nc);
  w.th = take(BH * w.nc * g.A);
  w.ddp = take(BH * w.nc);
  w.bias = take((size_t)w.nrb * 2 * g.H * g.N);
  w.total = off;
  return w;
}

size_t summary_lds_bytes(int PT, int NT) {
  const int NS = NT * 16 + 4, PS = PT * 16 + 4;
  return (size_t)(2 * BQ * NS + 2 * BQ * PS + 6 * BQ) * sizeof(float);
}

size_t group_lds_bytes(const ScanGeom& g) {
  const int HG = (int)(g.H / g.G), RN = (int)(g.R * g.N);
  const int nact = std::min(std::max(1, 256 / RN), HG);
  return (size_t)(2 * HG * RN + nact * 2 * RN) * sizeof(float);
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0u; }

void raise_lds(const void* fn, size_t bytes) {
  if (bytes > 64 * 1024 &&
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
    (void)hipGetLastError();
}

// The group reduction (8): 16-byte version when the layout allows it.
hipError_t launch_group(const ScanGeom& g, const BwdK& k, const BwdOperands& go, const void* workspace,
                        hipStream_t stream) {
  const unsigned C4 = (unsigned)(g.R * g.N / 4), HG = (unsigned)(g.H / g.G);
  if (g.N % 4u == 0 && aligned16(workspace) && aligned16(go.d_b) && aligned16(go.d_c)) {
    const unsigned nhs = std::min(std::max(1u, 256u / C4), HG);
    const size_t bytes = nhs > 1 ? (size_t)nhs * RB * C4 * 16 : 0;
    raise_lds(reinterpret_cast<const void*>(&bwd_group4_kernel), bytes);
    hipLaunchKernelGGL(bwd_group4_kernel, dim3(k.nrb, g.G), dim3(256), bytes, stream, k);
  } else {
    const size_t gl = group_lds_bytes(g);
    raise_lds(reinterpret_cast<const void*>(&bwd_group_kernel), gl);
    hipLaunchKernelGGL(bwd_group_kernel, dim3(k.nrb, g.G), dim3(256), gl, stream, k);
  }
  return hipGetLastError();
}

// The chunk prefix (4) over the summaries of mode (1: hs, 2: gs, 3: both).
hipError_t launch_prefix(const ScanGeom& g, const BwdK& k, int mode, const void* workspace, hipStream_t stream) {
  const unsigned BH = g.B * g.H, PN = g.P * g.N, ndir = mode == 3 ? 2u : 1u;
  if (PN % 4u == 0 && aligned16(workspace)) {
    const unsigned nb = (PN / 4u + 255u) / 256u;
    hipLaunchKernelGGL(bwd_prefix_kernel<4>, dim3(nb * BH, ndir), dim3(256), 0, stream, k, (int)nb, mode);
  } else {
    const unsigned nb = (PN + 255u) / 256u;
    hipLaunchKernelGGL(bwd_prefix_kernel<1>, dim3(nb * BH, ndir), dim3(256), 0, stream, k, (int)nb, mode);
  }
  return hipGetLastError();
}


}  // namespace

size_t siso_bwd_workspace_floats(const ScanGeom& g) { return bwd_layout(g).total; }

bool siso_bwd_fits(const ScanGeom& g) {
  const int PT = (int)((g.P + 15) / 16), NT = (int)((g.N + 15) / 16);
  // per-thread item arrays of the chunk kernel: 32 x (N - A) <= 512 * 8 and 32 x 16 PT <= 512 * 8
  if (BQ * (int)(g.N - g.A) > 512 * KQ_ITEMS || BQ * PT * 16 > 512 * XG_ITEMS) return false;
  const size_t chunk = (size_t)chunk_lds(PT, NT, (int)g.A).total * sizeof(float);
  return chunk <= 160 * 1024 && summary_lds_bytes(PT, NT) <= 160 * 1024 && group_lds_bytes(g) <= 160 * 1024;
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
  k.theta = ws + w.theta; k.tpre = ws + w.tpre; k.hs = ws + w.hs; k.gs = ws + w.gs; k.decay = ws + w.decay;
  k.dtheta = ws + w.dtheta; k.db_head = ws + w.dbh; k.dc_head = ws + w.dch;
  k.dsv = ws + w.dsv; k.ev = ws + w.ev; k.phi_tot = ws + w.phi; k.th_tot = ws + w.th;
  k.dd_part = ws + w.ddp; k.bias_part = ws + w.bias;
  k.B = (int)g.B; k.L = (int)g.L; k.H = (int)g.H; k.G = (int)g.G; k.P = (int)g.P; k.N = (int)g.N;
  k.A = (int)g.A; k.has_z = (int)g.has_z; k.has_d = (int)g.has_d;
  k.R = 1; k.RS = 1; k.rsl = 0; k.Qt = BQ;
  k.nc = w.nc; k.nT = w.nT; k.NT = (int)((g.N + 15) / 16); k.PT = (int)((g.P + 15) / 16); k.nrb = w.nrb;
  const unsigned BH = g.B * g.H;
  hipError_t e;
  if (g.A > 0) {
    if (g.A <= 32)
      hipLaunchKernelGGL(bwd_theta_local32_kernel, dim3(BH * w.nT), dim3(64), 0, stream, k);
    else
      hipLaunchKernelGGL(bwd_theta_local_kernel, dim3(BH * w.nT), dim3(64), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_theta_scan_kernel, dim3(BH * g.A), dim3(64), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the N = 128 / P = 64 / A = 32 geometry with 16-byte aligned operands
  // takes the kernels specialised for it
  const bool fixed = g.N == 128 && g.P == 64 && g.A == 32 && aligned16(workspace) && aligned16(o.b) &&
                     aligned16(o.c) && aligned16(o.x) && aligned16(go.dout) && aligned16(o.b_bias) &&
                     aligned16(o.c_bias) && (!g.has_z || aligned16(o.z));
  const size_t sl = summary_lds_bytes(k.PT, k.NT);
  if (fixed) {
    raise_lds(reinterpret_cast<const void*>(&bwd_summary_kernel<128, 64, 32>), sl);
    hipLaunchKernelGGL((bwd_summary_kernel<128, 64, 32>), dim3(BH * w.nc), dim3(512), sl, stream, k);
  } else {
    raise_lds(reinterpret_cast<const void*>(&bwd_summary_kernel<0, 0, -1>), sl);
    hipLaunchKernelGGL((bwd_summary_kernel<0, 0, -1>), dim3(BH * w.nc), dim3(512), sl, stream, k);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_prefix(g, k, 3, workspace, stream)) != hipSuccess) return e;
  const size_t cl = (size_t)chunk_lds(k.PT, k.NT, k.A).total * sizeof(float);
  if (fixed) {
    raise_lds(reinterpret_cast<const void*>(&bwd_chunk_kernel<true, 128, 64, 32>), cl);
    hipLaunchKernelGGL((bwd_chunk_kernel<true, 128, 64, 32>), dim3(BH * w.nc), dim3(512), cl, stream, k);
  } else if ((g.N & 3u) == 0 && aligned16(workspace)) {
    raise_lds(reinterpret_cast<const void*>(&bwd_chunk_kernel<true, 0, 0, -1>), cl);
    hipLaunchKernelGGL((bwd_chunk_kernel<true, 0, 0, -1>), dim3(BH * w.nc), dim3(512), cl, stream, k);
  } else {
    raise_lds(reinterpret_cast<const void*>(&bwd_chunk_kernel<false, 0, 0, -1>), cl);
    hipLaunchKernelGGL((bwd_chunk_kernel<false, 0, 0, -1>), dim3(BH * w.nc), dim3(512), cl, stream, k);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_chunk_scan_kernel, dim3(BH * (g.A + 1)), dim3(64), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_apply_kernel, dim3(BH * ((g.L + 31) / 32)), dim3(256), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_group(g, k, go, workspace, stream)) != hipSuccess) return e;
  const unsigned nb = (2u * g.H * g.N + 63u) / 64u + (g.H + 63u) / 64u;
  hipLaunchKernelGGL(bwd_bias_kernel, dim3(nb), dim3(1024), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (g.A > 0) {
    const size_t tot = (size_t)g.B * g.L * g.A;
    hipLaunchKernelGGL(bwd_angle_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace m3

namespace m3 {
namespace {

struct MimoLayout {
  size_t theta, tpre, hs, gs, decay, dtheta, dbh, dch, gyr, rho, dsv, ev, phi, th, ddp, mx, mz, mo, nw, bias, total;
  int RS, rsl, Qt, nc, nT, nrb;
};

MimoLayout mimo_layout(const ScanGeom& g) {
  MimoLayout w{};
  w.RS = 1;
  while (w.RS < (int)g.R) w.RS <<= 1;
  w.rsl = 0;
  while ((1 << w.rsl) < w.RS) ++w.rsl;
  w.Qt = BQ / w.RS;
  const size_t BH = (size_t)g.B * g.H;
  w.nc = (int)((g.L + w.Qt - 1) / w.Qt);
  w.nT = (int)((g.L + TT - 1) / TT);
  w.nrb = (int)(((size_t)g.B * g.L + RB - 1) / RB);
  const size_t nch = BH * w.nc;
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t o = off;
    off += (n + 63) / 64 * 64;
    return o;
  };
  w.theta = take(BH * g.L * g.A);
  w.tpre = take(BH * w.nT * g.A);
  w.hs = take(nch * g.P * g.N);
  w.gs = take(nch * g.P * g.N);
  w.decay = take(nch);
  w.dtheta = take(BH * g.L * g.A);
  w.dbh = take((size_t)g.B * g.L * g.H * g.R * g.N);
  w.dch = take((size_t)g.B * g.L * g.H * g.R * g.N);
  w.gyr = take(nch * BQ * g.P);
  w.rho = take(BH * g.L);
  w.dsv = take(BH * g.L);
  w.ev = take(BH * g.L);
  w.phi = take(nch);
  w.th = take(nch * g.A);
  w.ddp = take(nch);
  w.mx = take(nch * g.R * g.P);
  w.mz = take(nch * g.R * g.P);
  w.mo = take(nch * g.R * g.P);
  w.nw = take(nch * g.P);
  w.bias = take((size_t)w.nrb * 2 * g.H * g.R * g.N);
  w.total = off;
  return w;
}

size_t mimo_summary_lds(int PT, int NT) {
  const int NS = NT * 16 + 4, PS = PT * 16 + 4;
  return (size_t)(2 * BQ * NS + BQ * PS + 6 * BQ) * sizeof(float);
}

template <bool VEC4, int RSC, int NC, int PC, int AC>
hipError_t launch_post_rs(const BwdK& k, unsigned nch, size_t pl, hipStream_t stream) {
  raise_lds(reinterpret_cast<const void*>(&mimo_post_kernel<VEC4, RSC, NC, PC, AC>), pl);
  hipLaunchKernelGGL((mimo_post_kernel<VEC4, RSC, NC, PC, AC>), dim3(nch), dim3(512), pl, stream, k);
  return hipGetLastError();
}

template <bool VEC4, int NC, int PC, int AC>
hipError_t launch_post(const BwdK& k, int RS, unsigned nch, size_t pl, hipStream_t stream) {
  switch (RS) {
    case 1: return launch_post_rs<VEC4, 1, NC, PC, AC>(k, nch, pl, stream);
    case 2: return launch_post_rs<VEC4, 2, NC, PC, AC>(k, nch, pl, stream);
    case 4: return launch_post_rs<VEC4, 4, NC, PC, AC>(k, nch, pl, stream);
    default: return launch_post_rs<VEC4, 8, NC, PC, AC>(k, nch, pl, stream);
  }
}

size_t mimo_post_lds(int PT, int NT, int RS, int R, int P, int Qt) {
  const int NS = NT * 16 + 4, PS = PT * 16 + 4;
  return (size_t)(2 * BQ * NS + 3 * BQ * PS + BQ * MS + 8 * RS * PT * 16 + 2 * R * P + P + 2 * Qt * P + 5 * BQ) *
         sizeof(float);
}

}  // namespace

size_t mimo_bwd_workspace_floats(const ScanGeom& g) { return mimo_layout(g).total; }

bool mimo_bwd_fits(const ScanGeom& g) {
  const MimoLayout w = mimo_layout(g);
  const int PT = (int)((g.P + 15) / 16), NT = (int)((g.N + 15) / 16);
  const size_t lim = 160 * 1024;
  const size_t chunk = (size_t)mimo_chunk_lds(PT, NT, (int)g.A, w.RS, w.Qt).total * sizeof(float);
  return w.RS <= 8 && chunk <= lim && mimo_post_lds(PT, NT, w.RS, (int)g.R, (int)g.P, w.Qt) <= lim && mimo_summary_lds(PT, NT) <= lim &&
         group_lds_bytes(g) <= lim;
}

hipError_t launch_mimo_bwd(const ScanGeom& g, const ScanOperands& o, const BwdOperands& go, void* workspace,
                           hipStream_t stream) {
  const MimoLayout w = mimo_layout(g);
  float* ws = static_cast<float*>(workspace);
  BwdK k{};
  k.dout = go.dout;
  k.c = o.c; k.b = o.b; k.x = o.x; k.z = o.z; k.adt = o.adt; k.dt = o.dt; k.trap = o.trap;
  k.angle = o.angle; k.c_bias = o.c_bias; k.b_bias = o.b_bias; k.d = o.d;
  k.mimo_x = o.mimo_x; k.mimo_z = o.mimo_z; k.mimo_o = o.mimo_o; k.norm_weight = o.norm_weight;
  k.d_c = go.d_c; k.d_b = go.d_b; k.d_x = go.d_x; k.d_z = go.d_z; k.d_adt = go.d_adt; k.d_dt = go.d_dt;
  k.d_trap = go.d_trap; k.d_angle = go.d_angle; k.d_c_bias = go.d_c_bias; k.d_b_bias = go.d_b_bias;
  k.d_d = go.d_d;
  k.d_mimo_x = go.d_mimo_x; k.d_mimo_z = go.d_mimo_z; k.d_mimo_o = go.d_mimo_o;
  k.d_norm_weight = go.d_norm_weight;
  k.theta = ws + w.theta; k.tpre = ws + w.tpre; k.hs = ws + w.hs; k.gs = ws + w.gs; k.decay = ws + w.decay;
  k.dtheta = ws + w.dtheta; k.db_head = ws + w.dbh; k.dc_head = ws + w.dch; k.gyr = ws + w.gyr;
  k.rho = ws + w.rho; k.dsv = ws + w.dsv; k.ev = ws + w.ev; k.phi_tot = ws + w.phi; k.th_tot = ws + w.th;
  k.dd_part = ws + w.ddp; k.mx_part = ws + w.mx; k.mz_part = ws + w.mz; k.mo_part = ws + w.mo;
  k.nw_part = ws + w.nw; k.bias_part = ws + w.bias;
  k.B = (int)g.B; k.L = (int)g.L; k.H = (int)g.H; k.G = (int)g.G; k.P = (int)g.P; k.N = (int)g.N;
  k.A = (int)g.A; k.has_z = (int)g.has_z; k.has_d = (int)g.has_d; k.has_norm = (int)g.has_norm;
  k.R = (int)g.R; k.RS = w.RS; k.rsl = w.rsl; k.Qt = w.Qt;
  k.nc = w.nc; k.nT = w.nT; k.NT = (int)((g.N + 15) / 16); k.PT = (int)((g.P + 15) / 16); k.nrb = w.nrb;
  const unsigned BH = g.B * g.H;
  const unsigned nch = BH * (unsigned)w.nc;
  hipError_t e;
  if (g.A > 0) {
    if (g.A <= 32)
      hipLaunchKernelGGL(bwd_theta_local32_kernel, dim3(BH * w.nT), dim3(64), 0, stream, k);
    else
      hipLaunchKernelGGL(bwd_theta_local_kernel, dim3(BH * w.nT), dim3(64), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_theta_scan_kernel, dim3(BH * g.A), dim3(64), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the N = 128 / P = 64 / A = 32 geometry with 16-byte aligned operands
  // takes the kernels specialised for it
  const MimoChunkLds cll = mimo_chunk_lds(k.PT, k.NT, k.A, w.RS, w.Qt);
  const bool fixed = g.N == 128 && g.P == 64 && g.A == 32 && aligned16(workspace) && aligned16(o.b) &&
                     aligned16(o.c) && aligned16(o.x) && aligned16(go.dout) && aligned16(o.b_bias) &&
                     aligned16(o.c_bias) && aligned16(o.mimo_x) && (!g.has_z || aligned16(o.z)) &&
                     cll.o_xt % 4 == 0 && cll.o_msg % 4 == 0 && cll.o_cs % 4 == 0 && cll.o_sn % 4 == 0;
  const size_t sl = mimo_summary_lds(k.PT, k.NT);
  if (fixed) {
    raise_lds(reinterpret_cast<const void*>(&mimo_summary_kernel<128, 64, 32>), sl);
    hipLaunchKernelGGL((mimo_summary_kernel<128, 64, 32>), dim3(nch), dim3(512), sl, stream, k);
  } else {
    raise_lds(reinterpret_cast<const void*>(&mimo_summary_kernel<0, 0, -1>), sl);
    hipLaunchKernelGGL((mimo_summary_kernel<0, 0, -1>), dim3(nch), dim3(512), sl, stream, k);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_prefix(g, k, 1, workspace, stream)) != hipSuccess) return e;
  const size_t pl = mimo_post_lds(k.PT, k.NT, w.RS, k.R, k.P, w.Qt);
  const bool vec4 = (g.N & 3u) == 0 && aligned16(workspace);  // 16-byte state rows
  if (fixed)
    e = launch_post<true, 128, 64, 32>(k, w.RS, nch, pl, stream);
  else if (vec4)
    e = launch_post<true, 0, 0, -1>(k, w.RS, nch, pl, stream);
  else
    e = launch_post<false, 0, 0, -1>(k, w.RS, nch, pl, stream);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_prefix(g, k, 2, workspace, stream)) != hipSuccess) return e;
  const size_t cl = (size_t)cll.total * sizeof(float);
  if (fixed) {
    raise_lds(reinterpret_cast<const void*>(&mimo_chunk_kernel<true, 128, 64, 32>), cl);
    hipLaunchKernelGGL((mimo_chunk_kernel<true, 128, 64, 32>), dim3(nch), dim3(512), cl, stream, k);
  } else if (vec4) {
    raise_lds(reinterpret_cast<const void*>(&mimo_chunk_kernel<true, 0, 0, -1>), cl);
    hipLaunchKernelGGL((mimo_chunk_kernel<true, 0, 0, -1>), dim3(nch), dim3(512), cl, stream, k);
  } else {
    raise_lds(reinterpret_cast<const void*>(&mimo_chunk_kernel<false, 0, 0, -1>), cl);
    hipLaunchKernelGGL((mimo_chunk_kernel<false, 0, 0, -1>), dim3(nch), dim3(512), cl, stream, k);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_chunk_scan_kernel, dim3(BH * (g.A + 1)), dim3(64), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_apply_kernel, dim3(BH * ((g.L + 31) / 32)), dim3(256), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_group(g, k, go, workspace, stream)) != hipSuccess) return e;
  const unsigned nb = (2u * g.H * g.R * g.N + 63u) / 64u + (g.H + 63u) / 64u;
  hipLaunchKernelGGL(bwd_bias_kernel, dim3(nb), dim3(1024), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned nwb = 3u * g.H * ((g.R * g.P + 63u) / 64u) + g.H * ((g.P + 63u) / 64u);
  hipLaunchKernelGGL(mimo_weights_kernel, dim3(nwb), dim3(1024), 0, stream, k);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (g.A > 0) {
    const size_t tot = (size_t)g.B * g.L * g.A;
    hipLaunchKernelGGL(bwd_angle_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, stream, k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace m3
