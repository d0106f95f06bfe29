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
//   * One workgroup runs one (batch, head, sequence segment).  MFMA wave
//     (pt, nh) owns the 16 head_dim columns [16 pt, 16 pt + 16) and the
//     state rows of N-part nh (at most 64 of the N state coordinates); it
//     keeps that slice of h'^T in MFMA accumulator registers for the whole
//     segment.  The N-parts' partial outputs meet in LDS.  The block has
//     enough waves that each thread prefetches at most two 16-byte B and C
//     vectors, so a wave fits in 128 VGPRs and four waves share each SIMD.
//   * Intra-chunk S = Q K^T, the decay/trapezoid mask, M X and the
//     carried-state read Q h'^T run on v_mfma_f32_16x16x4_f32.  The state
//     update K^T (w X) does too, except in the N = 128 / P = 64 variant
//     (SISO both passes, MIMO the summary pass), where it runs on
//     v_mfma_f32_16x16x32_bf16 with each fp32 operand split into three bf16
//     pieces and six products accumulated in fp32 (about 2^-23 relative
//     error per product, fp32 level): the fp32 matrix pipe issues through
//     the vector ALU on gfx950, bf16 products do not, and the update is a
//     third of the chunk's matrix work.
//   * The next chunk's x, B, C, angle and scalars are loaded into registers
//     while the current chunk's MFMA work runs; z is loaded at the start of
//     the chunk that uses it.  (The bf16-update variant issues the next x
//     and this chunk's z after S, where its registers allow.)  The
//     cumulative angle is a 32-lane scan.
//   * Sequence segments: a first pass computes the end state of each piece
//     (two per segment before the last) from a zero entry, plus its decay
//     product and angle increment, into the workspace; the main pass folds
//     the earlier pieces' summaries, in order, into its entry state, so the
//     segments of one sequence run in parallel.
#include "common.h"
#include "launch.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>

namespace m3 {
namespace {

constexpr int kAux = 68;        // per segment summary: angle increment [<=64], decay at 64
constexpr int kAuxDecay = 64;
constexpr float kNormEps = 1.0e-5f;  // MIMO output-norm epsilon of the MIMO push constants
constexpr int kQV = 32;         // virtual rows per chunk
constexpr long kMaxAutoSegments = 65;  // automatic plan: at most 64 summaries per chain (one per segment)
// Key buffer of the bf16 state update, transposed: per state coordinate n one
// row of 32 bf16 (16 words), its four 16-byte blocks stored in the order
// q ^ ((n >> 2) & 3), so that the 16 rows read by one lane group hit 16
// different bank groups.
constexpr int kKTw = 16;
// fp16 query / key planes of the main pass (HALF below): rows of 136
// halves (128 + 8 pad, 272 bytes), head plane then tail plane
constexpr int kPQK = 136;
// Column of state coordinate n in a plane row: within each group of 32,
// n = 16 u + 4 q + e (e < 4) goes to 8 q + 4 u + e, so that the eight
// coordinates lane group q holds of two adjacent 16-row state blocks
// (4 q .. 4 q + 3 of each) are contiguous: one 16-byte read per MFMA
// operand in the read-out.  S contracts over the same order on both sides.
__device__ __forceinline__ int colp(int n) {
  return (n & ~31) | (((n >> 2) & 3) << 3) | (((n >> 4) & 1) << 2) | (n & 3);
}

struct ScanKParams {
  const float *c, *b, *x, *z, *adt, *dt, *trap, *angle, *c_bias, *b_bias, *d;
  const float *mimo_x, *mimo_z, *mimo_o, *norm_weight;
  float* out;
  float* ws_state;  // [B*H][(nseg-1) npc][PT*NT tiles][64 lanes][4]
  float* ws_aux;    // [B*H][(nseg-1) npc][kAux]
  int B, L, H, G, P, N, A, R;
  int has_z, has_d, has_norm;
  int NT, PT;       // 16-wide blocks of N and P
  int NH, NTH;      // N split into NH parts of NTH 16-wide blocks (one part per wave)
  int RS, rs_log2;  // rank stride of the virtual rows (power of two >= R)
  int Qt;           // tokens per chunk (QV / RS)
  int xstr, tstr, astr;  // per-token strides of x / z, trap and angle (packed rows share one)
  int seg_len, nseg;
  int npc, plen;    // summary pieces per segment before the last, and their length (tokens)
  // LDS layout (float offsets) and row strides
  int o_ql, o_kl, o_kt, o_xl, o_ml, o_ml2, o_yl, o_yl2, o_cs, o_bias, o_mimo, o_sc, o_run, lds_floats;
  int ks, xs, ms, ys;
};

// Compile-time variants: the fixed-size one (block counts and wave count known)
// and, within it, the merged key/query layout (one 8-column group of the B / C
// rows per half-wave).
__host__ __device__ constexpr bool fixed_variant(int NTC, int PTC, int NWC) {
  return NTC > 0 && PTC > 0 && NWC > 0 && NTC % (NTC > 4 ? 2 : 1) == 0 && PTC * (NTC > 4 ? 2 : 1) == NWC;
}
__host__ __device__ constexpr bool merged_variant(int NTC, int PTC, int NWC, int RSC) {
  return fixed_variant(NTC, PTC, NWC) && NTC * 16 == 16 * NWC && RSC > 0;
}

// Two workgroups share a CU, and the wave arbiter, at equal priority,
// favours the older one, so the workgroup dispatched second runs its chunks
// markedly slower and finishes alone, at one workgroup's rate.  Each
// workgroup sets its waves' priority from the chunks it has left (more left,
// higher priority, in bins that narrow towards the end), so the one behind
// takes the issue slots and the two finish close together.
__device__ __forceinline__ void set_progress_priority(int left) {
  if (left > 6) __builtin_amdgcn_s_setprio(3);
  else if (left > 3) __builtin_amdgcn_s_setprio(2);
  else if (left > 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

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
__device__ __forceinline__ typename VecOf<VEC>::T bload(rsrc_t r, uint32_t elem_off) {
  if constexpr (VEC == 4)
    return buf_load4(r, elem_off * 4u);
  else
    return buf_load1(r, elem_off * 4u);
}
template <int VEC>
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t elem_off, const typename VecOf<VEC>::T& v) {
  if constexpr (VEC == 4)
    buf_store4(r, elem_off * 4u, v);
  else
    buf_store1(r, elem_off * 4u, v);
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

// NTC / PTC / NWC fix the 16-wide block counts of N and P and the number of
// waves at compile time (0 = taken from the parameters), so that LDS row
// strides are constants and accesses fold into immediate offsets; RSC fixes
// the rank stride of the virtual rows (0 = from the parameters).  Fixed-size
// variants ask for two resident workgroups per CU (NWC / 2 waves per SIMD,
// at most 128 VGPRs).  STR reads x / z, trap and angle with the per-token
// strides of the parameters (packed projection rows); otherwise they are
// dense and the strides are H P, H and A.
template <int VEC, bool FULL, bool MIMO, int NTC, int PTC, int NWC, int RSC, bool STR>
__global__ __launch_bounds__(NWC ? NWC * 64 : 1024, NWC ? NWC / 2 : 1) void scan_chunk_kernel(ScanKParams p) {
  using vec_t = typename VecOf<VEC>::T;
  constexpr int QV = kQV;
  constexpr int TB = QV / 16;
  constexpr int KX = VEC == 4 ? 1 : 4;  // x / z items per thread (block >= Qt*P/(VEC*KX) threads)
  constexpr int KB = VEC == 4 ? 2 : 8;  // B / C row items per thread (block >= QV*N/(VEC*KB) threads)
  constexpr int KA = 4;         // angle values per lane (launch gives >= A/8 waves)
  // tokens per wave in the MIMO epilogue (a chunk holds QV / RS tokens)
  constexpr int KZM = (RSC > 0 && NWC > 0) ? ((QV / RSC) > NWC ? (QV / RSC) / NWC : 1) : 8;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nthreads = NWC ? NWC * 64 : (int)blockDim.x;
  const int nwaves = nthreads >> 6;
  const int l16 = lane & 15;
  const int lq = lane >> 4;

  // the main pass runs (b, h, segment); the summary pass (b, h, piece), each
  // of the first nseg - 1 segments cut into npc pieces of plen tokens
  const int nsum_all = (p.nseg - 1) * p.npc;  // summaries per (b, h)
  const int nseg_run = FULL ? p.nseg : nsum_all;
  const uint32_t unit = xcd_remap(blockIdx.x, gridDim.x);
  const int h = unit % p.H;
  const int rest = unit / p.H;
  const int seg = rest % nseg_run;
  const int b = rest / nseg_run;
  const int g = h / (p.H / p.G);
  const int bh = b * p.H + h;
  const int seg_base = (FULL ? seg : seg / p.npc) * p.seg_len;
  const int piece = FULL ? 0 : seg - (seg / p.npc) * p.npc;
  const int t_begin = min(seg_base + piece * p.plen, p.L);
  const int t_end = FULL ? min(seg_base + p.seg_len, p.L) : min(seg_base + min((piece + 1) * p.plen, p.seg_len), p.L);
  const int nsum = FULL ? seg * p.npc : 0;  // summaries folded into the entry state
  const int R = MIMO ? p.R : 1;
  const int RG = R * p.G;
  const int Qt = MIMO ? p.Qt : QV;
  constexpr int RSL_C = RSC >= 8 ? 3 : RSC >= 4 ? 2 : RSC >= 2 ? 1 : 0;
  const int rsl = RSC > 0 ? RSL_C : (MIMO ? p.rs_log2 : 0);
  const int NT = NTC ? NTC : p.NT, PT = PTC ? PTC : p.PT;
  const int NH = NTC ? (NTC > 4 ? 2 : 1) : p.NH;
  const int NTH = NTC ? (NTC + NH - 1) / NH : p.NTH;
  const int N = NTC ? NTC * 16 : p.N, P = PTC ? PTC * 16 : p.P, A = p.A;
  const int ks = NT * 16 + 4, xs = PT * 16 + 4, ms = QV + 4, ys = PT * 16 + 4;
  // In the fixed-size variant every wave is an MFMA wave with NTH state
  // blocks, known at compile time, so the block loops carry no branches and
  // the scheduler can overlap LDS reads with MFMAs across them.
  constexpr bool FIXED = fixed_variant(NTC, PTC, NWC);
  const bool mma_wave = FIXED || wave < PT * NH;
  const int pt = wave % PT;             // head_dim block of this MFMA wave
  const int nb0 = (wave / PT) * NTH;    // first state block of this MFMA wave
  const int ntw = FIXED ? NTH : (mma_wave ? min(NTH, NT - nb0) : 0);
  constexpr int JMAX = FIXED ? (NTC > 4 ? NTC / 2 : NTC) : 4;  // state blocks per wave (bound)
  // Fixed-size SISO: every (wave, half-wave) owns one 8-column group of the
  // B / C rows (N / 8 == 2 * waves), either a rotated pair group
  // (a0..a0+3, a0+A..a0+A+3) or a plain group, and rotates it in registers;
  // S is split over six waves (three tile pairs x two N-halves).
  constexpr bool MERGED = merged_variant(NTC, PTC, NWC, RSC);
  const int sw = nwaves - 1;  // wave that computes the per-token scalars
  // The merged layout runs its state update on split matrix products with k
  // = the chunk's 32 virtual rows at fp32-level accuracy: in the summary
  // pass on bf16 MFMA with the six-term split (v_mfma_f32_16x16x32_bf16), in
  // the main pass on fp16 MFMA with head / tail splits (KT16 below).  Its
  // keys go to LDS split into planes and transposed, [n][slot].  In the main
  // pass they sit beside the fp16 query / key planes that S = Q K^T reads,
  // and the raw y buffers overlay the key planes, which are dead once S is
  // formed.  Lane
  // group q of an MFMA operand holds virtual rows 4q..4q+3 and 16+4q..16+4q+3
  // in its eight k-slots, so row v sits in slot position
  //     pos(v) = 8 ((v >> 2) & 3) + 4 (v >> 4) + (v & 3)
  // of its key row, and the x rows a lane reads are 4 apart (16 banks apart).
  constexpr bool SPLIT = MERGED;
  // The main pass of the merged layout keeps its queries and keys as fp16
  // head / tail planes, split once by the lanes that rotate them, and forms
  // S = Q K^T and the read-out Q h'^T on v_mfma_f32_16x16x32_f16 from them
  // (three products per k = 32 step, about 2^-21 relative each).  The scales
  // are powers of two from a bound known before the rotation: the largest
  // raw B / C entry of the chunk plus the largest bias entry, times sqrt(2)
  // (a rotation keeps each pair's norm).
  constexpr bool HALF = FULL && MERGED;
  // The main pass keeps the transposed keys as two fp16 planes (head / tail
  // at the chunk's key scale) and splits w x per head_dim column: three fp16
  // products per state tile, their sum scaled back by a power of two and
  // added to the decayed state in one fused multiply-add
  constexpr bool KT16 = HALF;

  float* Ql = lds + p.o_ql;   // [QV][ks] C (+bias), pairs rotated in place   (main pass)
  float* Kl = lds + p.o_kl;   // [QV][ks] B (+bias), pairs rotated in place
  // HALF: the same regions as fp16 planes [head, tail][QV][kPQK]
  _Float16* const Qp = reinterpret_cast<_Float16*>(Ql);
  _Float16* const Kp = reinterpret_cast<_Float16*>(Kl);
  constexpr int QPL = QV * kPQK;  // halves per plane
  float* Xl = lds + p.o_xl;   // [QV][xs] per-rank x
  float* Ml = lds + p.o_ml;   // [QV][ms] masked S (N-half 0 when S is split)  (main pass)
  float* Ml2 = lds + p.o_ml2;  // [QV][ms] masked S, N-half 1 (split S only)
  float* Yl = lds + p.o_yl;   // [QV][ys] raw y, N-part 0 (+ M X)              (main pass)
  float* Yl2 = lds + p.o_yl2;  // [QV][ys] raw y, N-part 1                      (main pass)
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
  float* run = lds + p.o_run;  // [0,64) running theta, [64] chunk decay, [68] / [69] raw B / C maxima (HALF)
  unsigned* KTh = reinterpret_cast<unsigned*>(lds + p.o_kt);  // [N][kKTw] bf16 pairs of K, head parts (SPLIT)
  unsigned* KTm = KTh + N * kKTw;                     // middle parts
  unsigned* KTl = KTm + N * kKTw;                     // tail parts

  float seg_decay = 1.f;  // lane 0 of the scalar wave: product of chunk decays (summary pass)

  // ---- register prefetch of one chunk's global operands -------------------
  // Each operand is read through a buffer resource that starts at the chunk's
  // first token and ends after its last valid one, so rows past the end of
  // the chunk (or past the last item) load as zero without a branch.
  const int xrow = P / VEC;   // x items per token
  const int brow = N / VEC;   // B / C items per virtual row
  const int tokx = p.H * P;   // out elements per token
  const int tokxs = STR ? p.xstr : tokx;  // x / z elements per token
  const int astr = STR ? p.astr : A;      // angle elements per token
  const int tokb = RG * N;    // B / C elements per token
  vec_t xr[KX], br[KB], cr[KB];
  float angr[KA];
  float s_dt = 0.f, s_adt = 0.f, s_trap = 0.f;
  // merged layout: this lane's virtual row (token mtok, rank mr) and 8-column
  // group of the B / C rows; rows of padding ranks (mr >= R) stay zero
  const int mt = lane & 31;
  const int mtok = mt >> rsl;
  const int mr = mt & ((1 << rsl) - 1);
  const int mrc = mr < R ? mr : 0;  // a rank that exists, for addressing
  const int mgrp = 2 * wave + (lane >> 5);
  const bool mpair = MERGED && mgrp < A / 4;
  const int mc0 = mpair ? 4 * mgrp : 2 * A + 8 * (mgrp - A / 4);
  const int mc1 = mpair ? mc0 + A : mc0 + 4;
  float mdt = 0.f;

  // x rows of the chunk at token cs
  auto prefetch_x = [&](int cs) {
    const int nv = max(0, min(Qt, t_end - cs));  // 0 past the end: every load returns zero
    const rsrc_t xres = make_rsrc(STR ? p.x + ((size_t)b * p.L + cs) * tokxs + (size_t)h * P
                                      : p.x + (((size_t)b * p.L + cs) * p.H + h) * P,
                                  (uint32_t)(nv * tokxs * 4));
#pragma unroll
    for (int k = 0; k < KX; ++k) {
      const int idx = tid + k * nthreads;
      const int t = idx / xrow, pv = idx - t * xrow;
      xr[k] = bload<VEC>(xres, (uint32_t)(t * tokxs + pv * VEC));
    }
  };
  // The main pass with the split update is short of registers across S, so it
  // issues the next chunk's x loads after S (they land during the read-out,
  // the update and the epilogue); the other variants load x with the rest.
  constexpr bool LATE_X = FULL && SPLIT;
  auto prefetch = [&](int cs) {
    const int nv = max(0, min(Qt, t_end - cs));  // 0 past the end: every load returns zero
    const rsrc_t bres = make_rsrc(p.b + ((size_t)b * p.L + cs) * tokb, (uint32_t)(nv * tokb * 4));
    const rsrc_t cres = make_rsrc(p.c + ((size_t)b * p.L + cs) * tokb, (uint32_t)(nv * tokb * 4));
    const rsrc_t ares = make_rsrc(p.angle + ((size_t)b * p.L + cs) * astr, (uint32_t)(nv * astr * 4));
    if constexpr (!LATE_X) prefetch_x(cs);
    if constexpr (MERGED) {
      const uint32_t row = (uint32_t)(mtok * tokb + (mrc * p.G + g) * N);
      br[0] = bload<VEC>(bres, row + mc0);
      br[1] = bload<VEC>(bres, row + mc1);
      if (FULL) {
        cr[0] = bload<VEC>(cres, row + mc0);
        cr[1] = bload<VEC>(cres, row + mc1);
      }
      if (mpair) {
        // the offset is formed here each time rather than kept in a register
        // across the chunk loop (kept, it was spilled, and its reload waited
        // for every load in flight, the prefetch just issued included)
        int arow = mtok;
        asm volatile("" : "+v"(arow));
        const floatx4 a4 = buf_load4(ares, (uint32_t)(arow * astr + mc0) * 4u);
        angr[0] = a4.x; angr[1] = a4.y; angr[2] = a4.z; angr[3] = a4.w;
      }
      const size_t sbase = ((size_t)b * p.L + cs) * p.H + h;
      mdt = buf_load1(make_rsrc(p.dt + sbase, (uint32_t)(nv * p.H * 4)), (uint32_t)(mtok * p.H) * 4u);
    } else {
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int idx = tid + k * nthreads;
        const int u = idx / brow, j = idx - u * brow;
        const int t = u / R, r = u - t * R;
        const uint32_t off = (uint32_t)(t * tokb + (r * p.G + g) * N + j * VEC);
        br[k] = bload<VEC>(bres, off);
        if (FULL) cr[k] = bload<VEC>(cres, off);
      }
#pragma unroll
      for (int i = 0; i < KA; ++i) {
        const int a = 2 * (i * nwaves + wave) + (lane >> 5);
        const int t = lane & 31;
        angr[i] = a < A ? buf_load1(ares, (uint32_t)(t * astr + a) * 4u) : 0.f;
      }
    }
    if (wave == (MERGED ? sw : 0)) {
      // tokens cs .. cs + Qt (one past the chunk, for the trapezoid look-ahead)
      const size_t sbase = ((size_t)b * p.L + cs) * p.H + h;
      const uint32_t nl = (uint32_t)max(0, min(Qt + 1, p.L - cs));
      const rsrc_t dres = make_rsrc(p.dt + sbase, nl * p.H * 4);
      const rsrc_t tres = STR ? make_rsrc(p.trap + ((size_t)b * p.L + cs) * p.tstr + h, nl * p.tstr * 4)
                              : make_rsrc(p.trap + sbase, nl * p.H * 4);
      const rsrc_t adres = make_rsrc(p.adt + sbase, (uint32_t)(nv * p.H * 4));
      const uint32_t so = (uint32_t)(lane * p.H) * 4u;
      s_dt = buf_load1(dres, so);
      int tl = lane;  // (formed here each time, as the angle offset above)
      asm volatile("" : "+v"(tl));
      s_trap = buf_load1(tres, STR ? (uint32_t)(tl * p.tstr) * 4u : so);
      s_adt = buf_load1(adres, so);
    }
  };

  // The first chunk's loads go out before the set-up below (LDS clearing, biases,
  // the entry-state fold), whose own loads and waits they overlap.
  prefetch(t_begin);
  if constexpr (LATE_X) prefetch_x(t_begin);

  for (int i = tid; i < p.lds_floats; i += nthreads) lds[i] = 0.f;
  __syncthreads();
  for (int i = tid; i < R * N; i += nthreads) {
    bbL[i] = p.b_bias[(size_t)h * R * N + i];
    if (FULL) cbL[i] = p.c_bias[(size_t)h * R * N + i];
  }
  // HALF: the largest bias magnitudes of this head (with the raw-row maxima,
  // the bound behind the fp16 scales)
  float bmax_b = 0.f, bmax_c = 0.f;
  if constexpr (HALF) {
    for (int i = lane; i < R * N; i += 64) {
      bmax_b = max3_abs(p.b_bias[(size_t)h * R * N + i], 0.f, bmax_b);
      bmax_c = max3_abs(p.c_bias[(size_t)h * R * N + i], 0.f, bmax_c);
    }
    bmax_b = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max_nn(bmax_b))));
    bmax_c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max_nn(bmax_c))));
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

  const int p0 = pt * 16;
  floatx4 Hacc[4];  // state blocks nb0 .. nb0 + ntw - 1 of columns p0 .. p0 + 15
#pragma unroll
  for (int j = 0; j < JMAX; ++j) Hacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Entry state: fold the summaries of the earlier segments, in order,
  //   h' <- decay_i h' + rot(theta_i) U_i,
  // where U_i was built with the angle restarted at zero inside segment i, so
  // its state axis is turned by theta_i = the summed angle of the segments
  // before i (the keys it holds are rot(theta_i + local) = rot(theta_i) rot(local)).
  //
  // With N = 128 split into two halves of 64 state rows per wave and A a
  // multiple of 16 with 2A <= 64, both members of every rotated pair
  // (a, a + A) sit in the same lane and register of one wave (blocks a / 16
  // and a / 16 + A / 16), so the fold rotates in registers, with all
  // summaries loaded at once and cos / sin of every theta_i from an LDS table.
  // Otherwise U_i passes through LDS in [p][n] layout for the pair rotation.
  const bool reg_fold = FIXED && NTC == 8 && !MIMO && (A == 0 || A == 16 || A == 32) && nsum_all <= 128;
  if (FULL && seg > 0 && reg_fold) {
    const size_t sbase = (size_t)bh * nsum_all;
    // LDS (overlaying the chunk buffers, unused yet): the summaries' angle
    // increments and decays, loaded at once; then per angle the running sums
    // theta_i (in summary order), and cos / sin of each
    float* CSt = lds;  // [nsum][A] theta_i, then cos theta_i
    float* SNt = CSt + nsum * A;  // [nsum][A] sin theta_i
    float* AXt = SNt + nsum * A;  // [nsum][A] angle increment of summary i
    float* DCt = AXt + nsum * A;  // [nsum] decay of summary i
    for (int idx = tid; idx < nsum * A; idx += nthreads) {
      const int i = idx / A, a = idx - i * A;
      AXt[idx] = p.ws_aux[(sbase + i) * kAux + a];
    }
    for (int i = tid; i < nsum; i += nthreads) DCt[i] = p.ws_aux[(sbase + i) * kAux + kAuxDecay];
    __syncthreads();
    for (int a = tid; a < A; a += nthreads) {
      float th = 0.f;
      for (int i = 0; i < nsum; ++i) {
        CSt[i * A + a] = th;
        th += AXt[i * A + a];
      }
      run[a] = th;
    }
    __syncthreads();
    for (int idx = tid; idx < nsum * A; idx += nthreads) {
      float sn, cs;
      sincos_acc(CSt[idx], &sn, &cs);
      CSt[idx] = cs;
      SNt[idx] = sn;
    }
    __syncthreads();
    // the summary states, two in flight at a time (with the first chunk's
    // loads already in flight, four spill registers)
    constexpr int FB = 2;
    for (int i0 = 0; i0 < nsum; i0 += FB) {
      floatx4 u[FB][JMAX];
#pragma unroll
      for (int k = 0; k < FB; ++k) {
        if (i0 + k < nsum) {
          const float* st = p.ws_state + (sbase + i0 + k) * (size_t)(PT * NT) * 256;
#pragma unroll
          for (int j = 0; j < JMAX; ++j)
            u[k][j] = *reinterpret_cast<const floatx4*>(st + ((pt * NT + nb0 + j) * 64 + lane) * 4);
        }
      }
#pragma unroll
      for (int k = 0; k < FB; ++k) {
        const int i = i0 + k;
        if (i < nsum) {
          if (nb0 == 0 && A > 0) {
            const float* ci = CSt + i * A;
            const float* si = SNt + i * A;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (A == 32) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                  const int a = 16 * jb + 4 * lq + r;
                  const float c = ci[a], sv = si[a];
                  const float u0 = u[k][jb][r], u1 = u[k][jb + 2][r];
                  u[k][jb][r] = u0 * c - u1 * sv;
                  u[k][jb + 2][r] = u0 * sv + u1 * c;
                }
              } else {  // A == 16
                const int a = 4 * lq + r;
                const float c = ci[a], sv = si[a];
                const float u0 = u[k][0][r], u1 = u[k][1][r];
                u[k][0][r] = u0 * c - u1 * sv;
                u[k][1][r] = u0 * sv + u1 * c;
              }
            }
          }
          const float dec = DCt[i];
#pragma unroll
          for (int j = 0; j < JMAX; ++j) Hacc[j] = dec * Hacc[j] + u[k][j];
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < 3 * nsum * A + nsum; i += nthreads) CSt[i] = 0.f;  // restore the zeroed chunk buffers
  } else if (FULL && seg > 0) {
    __syncthreads();
    float* Ub = lds;  // [PT*16][NT*16 + 4], overlays the chunk buffers (unused yet)
    const int us = NT * 16 + 4;
    for (int i = 0; i < nsum; ++i) {
      const size_t si = (size_t)bh * nsum_all + i;
      const float* aux = p.ws_aux + si * kAux;
      const float* st = p.ws_state + si * (size_t)(PT * NT) * 256;
      if (mma_wave) {
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
          if (FIXED || j < ntw) {
            const int nb = nb0 + j;
            const floatx4 u = *reinterpret_cast<const floatx4*>(st + ((pt * NT + nb) * 64 + lane) * 4);
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
      for (int e = tid; e < PT * 16 * A; e += nthreads) {
        const int pp = e / A, a = e - pp * A;
        const float u0 = Ub[pp * us + a], u1 = Ub[pp * us + a + A];
        Ub[pp * us + a] = u0 * CS[a] - u1 * SN[a];
        Ub[pp * us + a + A] = u0 * SN[a] + u1 * CS[a];
      }
      __syncthreads();
      const float dec = aux[kAuxDecay];
      if (mma_wave) {
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
          if (FIXED || j < ntw) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              Hacc[j][r] = fmaf(dec, Hacc[j][r], Ub[(p0 + l16) * us + (nb0 + j) * 16 + 4 * lq + r]);
          }
        }
      }
      if (tid < A) run[tid] += aux[tid];
      __syncthreads();
    }
    for (int i = tid; i < PT * 16 * us; i += nthreads) Ub[i] = 0.f;  // restore the zero padding
  }
  // HALF: the largest raw B / C entries of the prefetched rows of a chunk,
  // for the staging of that chunk: each wave's maximum goes into one LDS
  // slot per operand by an integer atomic max (the values are non-negative,
  // so their bit patterns order as the floats do); the scalar wave clears
  // the slots during S, after the staging has read them
  auto raw_maxima = [&]() {
    if constexpr (HALF) {
      float mk = 0.f, mq = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        mk = max3_abs(br[i][0], br[i][1], mk);
        mk = max3_abs(br[i][2], br[i][3], mk);
        mq = max3_abs(cr[i][0], cr[i][1], mq);
        mq = max3_abs(cr[i][2], cr[i][3], mq);
      }
      mk = wave_max_nn(mk);
      mq = wave_max_nn(mq);
      if (lane == 0) {
        atomicMax(reinterpret_cast<unsigned*>(run + 68), __float_as_uint(mk));
        atomicMax(reinterpret_cast<unsigned*>(run + 69), __float_as_uint(mq));
      }
    }
  };
  auto slot_max = [&](const float* sl) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(*sl)));
  };
  // fp16 scale exponents of the staged chunk's keys and queries (uniform)
  int eK = 0, eQ = 0;
  // the D skip of this head, read once (read in the chunk loop, its load
  // came after the prefetches in flight and waited for all of them)
  const float dh = (FULL && p.has_d) ? __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(p.d[h]))) : 0.f;

  raw_maxima();
  __syncthreads();

  for (int c0 = t_begin; c0 < t_end; c0 += Qt) {
    const int nvalid = min(Qt, t_end - c0);
    if constexpr (FULL) set_progress_priority((t_end - c0 + Qt - 1) / Qt);

    // ---- P0: scalars (one wave, lane = token); x, B, C rows into LDS; z loads --
    if (wave == (MERGED ? sw : 0)) {
      const int t = lane;
      const float dt_n = next_lane_f(s_dt);
      const float tr_n = next_lane_f(s_trap);
      const bool ok = t < nvalid;
      const float dt_v = ok ? s_dt : 0.f;
      const float adt_v = ok ? s_adt : 0.f;
      const float gam = ok ? sigmoid_fast(s_trap) * dt_v : 0.f;
      float scl = gam;
      if (ok && c0 + t + 1 < p.L) scl = gam + (1.f - sigmoid_fast(tr_n)) * dt_n;
      const float cum = scan64_f(adt_v);
      const float cum_last = read_lane_f(cum, 63);  // padding lanes add zero
      if (t < Qt) {
        sc_cum[t] = cum;
        sc_ecum[t] = exp_fast(cum);
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
    if constexpr (MERGED) {
      // cumulative angle of this lane's token for four pair angles (DPP scans
      // over the 32 virtual rows of the half-wave; only rank 0 rows add, so
      // every rank of a token sees that token's angle), then the rotation in
      // registers
      const bool tok_ok = mtok < nvalid && mr < R;
      if constexpr (HALF) {
        // |rotated entry| <= sqrt(2) max |raw + bias| (a rotation keeps each pair's norm)
        eK = __builtin_amdgcn_readfirstlane(f16_scale_exp(1.4143f * (slot_max(run + 68) + bmax_b)));
        eQ = __builtin_amdgcn_readfirstlane(f16_scale_exp(1.4143f * (slot_max(run + 69) + bmax_c)));
      }
      float th[4] = {0.f, 0.f, 0.f, 0.f};
      if (2 * wave < A / 4) {  // the wave holds rotated pair groups (uniform)
#pragma unroll
        for (int e = 0; e < 4; ++e) th[e] = scan32_f((mpair && tok_ok && mr == 0) ? mdt * angr[e] : 0.f);
      }
      vec_t k0 = br[0], k1 = br[1], q0 = cr[0], q1 = cr[1];
      const float* bbr = bbL + mrc * N;
      const floatx4 bb0 = lds_read4(bbr + mc0), bb1 = lds_read4(bbr + mc1);
      k0 += bb0;
      k1 += bb1;
      if (FULL) {
        const float* cbr = cbL + mrc * N;
        q0 += lds_read4(cbr + mc0);
        q1 += lds_read4(cbr + mc1);
      }
      if (mpair) {
        const floatx4 r4 = lds_read4(run + mc0);
        float thv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          thv[e] = r4[e] + th[e];
          float sn, co;
          sincos_hw(thv[e], &sn, &co);
          const float u0 = k0[e], u1 = k1[e];
          k0[e] = u0 * co - u1 * sn;
          k1[e] = u0 * sn + u1 * co;
          if (FULL) {
            const float w0 = q0[e], w1 = q1[e];
            q0[e] = w0 * co - w1 * sn;
            q1[e] = w0 * sn + w1 * co;
          }
        }
        if (mt == ((nvalid - 1) << rsl)) *reinterpret_cast<floatx4*>(run + mc0) = floatx4{thv[0], thv[1], thv[2], thv[3]};
      }
      // rows past the chunk's last token, or of padding ranks (a full SISO
      // chunk has none: uniform test first)
      if ((nvalid < Qt || R < (1 << rsl)) && !tok_ok) {
        k0 = floatx4{0.f, 0.f, 0.f, 0.f};
        k1 = k0;
        q0 = k0;
        q1 = k0;
      }
      if constexpr (HALF) {
        // fp16 head / tail words of the four columns at mc0 and at mc1, in
        // the plane column order colp
        const float sK = ldexpf(1.f, eK), sQ = ldexpf(1.f, eQ);
        const int r0 = mt * kPQK + colp(mc0), r1 = mt * kPQK + colp(mc1);
        unsigned h0, h1, t0, t1;
        split2_f16s(k0[0], k0[1], sK, h0, t0);
        split2_f16s(k0[2], k0[3], sK, h1, t1);
        *reinterpret_cast<uintx2*>(Kp + r0) = uintx2{h0, h1};
        *reinterpret_cast<uintx2*>(Kp + QPL + r0) = uintx2{t0, t1};
        split2_f16s(k1[0], k1[1], sK, h0, t0);
        split2_f16s(k1[2], k1[3], sK, h1, t1);
        *reinterpret_cast<uintx2*>(Kp + r1) = uintx2{h0, h1};
        *reinterpret_cast<uintx2*>(Kp + QPL + r1) = uintx2{t0, t1};
        split2_f16s(q0[0], q0[1], sQ, h0, t0);
        split2_f16s(q0[2], q0[3], sQ, h1, t1);
        *reinterpret_cast<uintx2*>(Qp + r0) = uintx2{h0, h1};
        *reinterpret_cast<uintx2*>(Qp + QPL + r0) = uintx2{t0, t1};
        split2_f16s(q1[0], q1[1], sQ, h0, t0);
        split2_f16s(q1[2], q1[3], sQ, h1, t1);
        *reinterpret_cast<uintx2*>(Qp + r1) = uintx2{h0, h1};
        *reinterpret_cast<uintx2*>(Qp + QPL + r1) = uintx2{t0, t1};
      } else if (FULL || !SPLIT) {
        vstore<VEC>(Kl + mt * ks + mc0, k0);
        vstore<VEC>(Kl + mt * ks + mc1, k1);
      }
      if constexpr (SPLIT) {
        // Lanes 2i, 2i + 1 (virtual rows mt, mt + 1) trade halves so that each
        // writes one word (row mt, row mt + 1) for four columns: the even lane
        // for its columns mc0.., the odd lane for its columns mc1..  The head
        // plane goes first, then the middle and tail planes of the remainders.
        const bool odd = (mt & 1) != 0;
        const int col = odd ? mc1 : mc0;
        // word pos(mt & ~1) / 2 of the row: block (mt >> 2) & 3, swizzled by
        // the row (the same for the four rows col..col + 3), word 2 (mt >> 4) + ((mt >> 1) & 1)
        const int wd = 4 * (((mt >> 2) & 3) ^ ((col >> 2) & 3)) + 2 * (mt >> 4) + ((mt >> 1) & 1);
        // The even lane keeps its columns mc0.. and takes the odd lane's values
        // there; the odd lane keeps mc1.. and takes the even lane's: after one
        // exchange each lane holds rows mt & ~1 (ra) and mt | 1 (rb) of its
        // four columns, and each converted pair is one word of the plane.
        float ra[4], rb[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float own = odd ? k1[c] : k0[c];
          const float other = __uint_as_float(swap_pair_u(__float_as_uint(odd ? k0[c] : k1[c])));
          ra[c] = odd ? other : own;
          rb[c] = odd ? own : other;
        }
        if constexpr (KT16) {
          // fp16 head / tail planes at the chunk's key scale
          const float sK = ldexpf(1.f, eK);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            unsigned hw, lw;
            split2_f16s(ra[c], rb[c], sK, hw, lw);
            KTh[(col + c) * kKTw + wd] = hw;
            KTm[(col + c) * kKTw + wd] = lw;
          }
        } else {
#pragma unroll
          for (int part = 0; part < 3; ++part) {
            unsigned* dst = KTh + part * N * kKTw + col * kKTw + wd;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const unsigned w = __builtin_bit_cast(unsigned, __builtin_convertvector((floatx2){ra[c], rb[c]}, bf16x2));
              dst[c * kKTw] = w;
              if (part < 2) {  // the remainders for the next plane
                ra[c] -= __uint_as_float(w << 16);
                rb[c] -= __uint_as_float(w & 0xffff0000u);
              }
            }
          }
        }
      }
      if (FULL && !HALF) {
        vstore<VEC>(Ql + mt * ks + mc0, q0);
        vstore<VEC>(Ql + mt * ks + mc1, q1);
      }
    }
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int idx = tid + k * nthreads;
      if (!MERGED && idx < Qt * R * brow) {
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
    const size_t cbase_tok = (((size_t)b * p.L + c0) * p.H + h) * P;  // out at token c0
    // z and out: valid tokens of this chunk only (no z reads when has_z is off)
    const rsrc_t zres = make_rsrc(STR ? p.z + ((size_t)b * p.L + c0) * tokxs + (size_t)h * P : p.z + cbase_tok,
                                  p.has_z ? (uint32_t)(nvalid * tokxs * 4) : 0u);
    const rsrc_t ores = make_rsrc(p.out + cbase_tok, (uint32_t)(nvalid * tokx * 4));
    auto load_z = [&]() {
#pragma unroll
      for (int k = 0; k < KX; ++k) {
        const int idx = tid + k * nthreads;
        const int t = idx / xrow, pv = idx - t * xrow;
        zr[k] = bload<VEC>(zres, (uint32_t)(t * tokxs + pv * VEC));
      }
    };
    // MIMO: z of the tokens this wave finishes in the epilogue
    auto load_zm = [&]() {
#pragma unroll
      for (int i = 0; i < KZM; ++i) {
        const int t = wave + i * nwaves;
        const uint32_t ob = (uint32_t)(t * tokxs);
        zm[i][0] = lane < P ? buf_load1(zres, (ob + lane) * 4u) : 0.f;
        zm[i][1] = lane + 64 < P ? buf_load1(zres, (ob + lane + 64) * 4u) : 0.f;
      }
    };
    // With the split update the z loads wait until S is formed (the registers
    // are short across S); they land during the read-out and update.
    if constexpr (FULL && !MIMO && !SPLIT) load_z();
    if constexpr (FULL && MIMO && !SPLIT) load_zm();
    if constexpr (!MERGED) lds_barrier();

    // ---- P2: cumulative angle (32-lane scans), cos / sin, and the rotation of
    //      the pairs (a, a + A) of every rank's key and query row, in place -----
#pragma unroll
    for (int i = 0; i < (MERGED ? 0 : KA); ++i) {
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
    // Issued after the last chunk too (on empty ranges: no memory access,
    // zeros): with no branch around the loads the compiler counts them
    // through the loop and waits for exactly the ones it needs.
    prefetch(c0 + Qt);
    lds_barrier();

    if constexpr (FULL) {
      // ---- P4: S = Q K^T on lower 16x16 tiles, masked ------------------------
      constexpr int NPAIRS = TB * (TB + 1) / 2;
      // split S: unit = (tile pair, N-half), each masked into its own buffer
      constexpr int SPL = MERGED ? 2 : 1;
      for (int un = wave; un < NPAIRS * SPL; un += nwaves) {
        const int pr = un / SPL, half = un - pr * SPL;
        int tb = 0, sb = pr;
        while (sb > tb) { sb -= tb + 1; ++tb; }
        float* Mdst = half ? Ml2 : Ml;
        floatx4 acc;
        if constexpr (HALF) {
          // the N-half's 64 plane columns in two k = 32 steps, each the two
          // tail products, then the head product
          floatx4 a16 = floatx4{0.f, 0.f, 0.f, 0.f};
          const _Float16* qa = Qp + (tb * 16 + l16) * kPQK + half * 64 + 8 * lq;
          const _Float16* kb = Kp + (sb * 16 + l16) * kPQK + half * 64 + 8 * lq;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uintx4 qh = *reinterpret_cast<const uintx4*>(qa + 32 * i);
            const uintx4 ql = *reinterpret_cast<const uintx4*>(qa + QPL + 32 * i);
            const uintx4 kh = *reinterpret_cast<const uintx4*>(kb + 32 * i);
            const uintx4 kl = *reinterpret_cast<const uintx4*>(kb + QPL + 32 * i);
            a16 = mfma_f16(ql, kh, a16);
            a16 = mfma_f16(qh, kl, a16);
            a16 = mfma_f16(qh, kh, a16);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = ldexpf(a16[r], -(eQ + eK));
        } else {
          floatx4 accs[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
          const float* qa = Ql + (tb * 16 + l16) * ks + 4 * lq + half * (NT / SPL) * 16;
          const float* kb = Kl + (sb * 16 + l16) * ks + 4 * lq + half * (NT / SPL) * 16;
#pragma unroll
          for (int nb = 0; nb < 8 / SPL; ++nb) {
            if (nb < NT / SPL) {
              const floatx4 a4 = lds_read4(qa + nb * 16);
              const floatx4 b4 = lds_read4(kb + nb * 16);
              floatx4& ac = accs[nb & 1];
              ac = mfma16(a4.x, b4.x, ac);
              ac = mfma16(a4.y, b4.y, ac);
              ac = mfma16(a4.z, b4.z, ac);
              ac = mfma16(a4.w, b4.w, ac);
            }
          }
          acc = accs[0] + accs[1];
        }
        const int vs = sb * 16 + l16;
        const int ts_ = vs >> rsl;
        const float cum_s = sc_cum[ts_], scl_s = sc_scl[ts_];
        if constexpr (HALF) {
          // the weights of the lane's four rows by selects (every lane
          // computes the decay term; no branches)
          floatx4 cum_t, gam_t;
          if constexpr (RSC == 1) {  // one virtual row per token
            cum_t = lds_read4(sc_cum + tb * 16 + 4 * lq);
            gam_t = lds_read4(sc_gam + tb * 16 + 4 * lq);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              cum_t[r] = sc_cum[(tb * 16 + 4 * lq + r) >> rsl];
              gam_t[r] = sc_gam[(tb * 16 + 4 * lq + r) >> rsl];
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int vt = tb * 16 + 4 * lq + r;
            const int tt = vt >> rsl;
            float wdec = exp_fast(cum_t[r] - cum_s) * scl_s;
            asm volatile("" : "+v"(wdec));
            const float wt = ts_ < tt ? wdec : (ts_ == tt ? gam_t[r] : 0.f);
            Mdst[vt * ms + vs] = acc[r] * wt;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int vt = tb * 16 + 4 * lq + r;
            const int tt = vt >> rsl;
            float m = 0.f;
            if (ts_ < tt) m = acc[r] * (exp_fast(sc_cum[tt] - cum_s) * scl_s);
            else if (ts_ == tt) m = acc[r] * sc_gam[tt];
            Mdst[vt * ms + vs] = m;
          }
        }
      }
      if constexpr (HALF) {
        if (tid == sw * 64) *reinterpret_cast<floatx2*>(run + 68) = floatx2{0.f, 0.f};  // the staging has read them
      }
      lds_barrier();
    }

    if constexpr (FULL && !MIMO && SPLIT) load_z();
    if constexpr (FULL && MIMO && SPLIT) load_zm();
    if (mma_wave) {
      if constexpr (FULL) {
        // ---- P5a: Y = M X + diag(exp(cum)) Q h'^T over this wave's state
        //      blocks; N-part 0 adds the intra-chunk M X.
        // M X: Ml (+ Ml2) rows times the chunk's x.
        auto add_mx = [&](floatx4* acc) {
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            for (int sb = 0; sb <= tb; ++sb) {
              floatx4 a4 = lds_read4(Ml + (tb * 16 + l16) * ms + sb * 16 + 4 * lq);
              if constexpr (MERGED) a4 += lds_read4(Ml2 + (tb * 16 + l16) * ms + sb * 16 + 4 * lq);
              const float* xc = Xl + (sb * 16 + 4 * lq) * xs + p0 + l16;
              acc[tb] = mfma16(a4.x, xc[0], acc[tb]);
              acc[tb] = mfma16(a4.y, xc[xs], acc[tb]);
              acc[tb] = mfma16(a4.z, xc[2 * xs], acc[tb]);
              acc[tb] = mfma16(a4.w, xc[3 * xs], acc[tb]);
            }
          }
        };
        // Q h'^T, this wave's state blocks
        auto add_qh = [&](floatx4* aci) {
#pragma unroll
          for (int j = 0; j < JMAX; ++j) {
            if (FIXED || j < ntw) {
              const int nb = nb0 + j;
#pragma unroll
              for (int tb = 0; tb < TB; ++tb) {
                const floatx4 a4 = lds_read4(Ql + (tb * 16 + l16) * ks + nb * 16 + 4 * lq);
                aci[tb] = mfma16(a4.x, Hacc[j].x, aci[tb]);
                aci[tb] = mfma16(a4.y, Hacc[j].y, aci[tb]);
                aci[tb] = mfma16(a4.z, Hacc[j].z, aci[tb]);
                aci[tb] = mfma16(a4.w, Hacc[j].w, aci[tb]);
              }
            }
          }
        };
        float* Yd = nb0 == 0 ? Yl : Yl2;
        if constexpr (SPLIT) {
          // one accumulator set (this kernel is short of registers): Q h'^T,
          // its rows scaled by exp(cum), then M X accumulated on top
          floatx4 acc[TB];
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
          if constexpr (HALF) {
            // the state to fp16 head / tail, one scale per head_dim column
            // over this wave's state blocks; per pair of blocks (one k = 32
            // step, plane columns 32 i' .. 32 i' + 31 hold exactly their rows)
            // the two tail products, then the head product
            float hm = 0.f;
#pragma unroll
            for (int j = 0; j < JMAX; ++j) {
              hm = max3_abs(Hacc[j][0], Hacc[j][1], hm);
              hm = max3_abs(Hacc[j][2], Hacc[j][3], hm);
            }
            const int eH = f16_scale_exp(max_xor16_32(hm));
            const float sH = ldexpf(1.f, eH);
#pragma unroll
            for (int i = 0; i < JMAX / 2; ++i) {
              unsigned h0, h1, h2, h3, t0, t1, t2, t3;
              split2_f16s(Hacc[2 * i][0], Hacc[2 * i][1], sH, h0, t0);
              split2_f16s(Hacc[2 * i][2], Hacc[2 * i][3], sH, h1, t1);
              split2_f16s(Hacc[2 * i + 1][0], Hacc[2 * i + 1][1], sH, h2, t2);
              split2_f16s(Hacc[2 * i + 1][2], Hacc[2 * i + 1][3], sH, h3, t3);
              const uintx4 hh = uintx4{h0, h1, h2, h3}, hl = uintx4{t0, t1, t2, t3};
#pragma unroll
              for (int tb = 0; tb < TB; ++tb) {
                const _Float16* qr = Qp + (tb * 16 + l16) * kPQK + (nb0 + 2 * i) * 16 + 8 * lq;
                const uintx4 qh = *reinterpret_cast<const uintx4*>(qr);
                const uintx4 ql = *reinterpret_cast<const uintx4*>(qr + QPL);
                acc[tb] = mfma_f16(ql, hh, acc[tb]);
                acc[tb] = mfma_f16(qh, hl, acc[tb]);
                acc[tb] = mfma_f16(qh, hh, acc[tb]);
              }
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[tb][r] = ldexpf(acc[tb][r], -(eQ + eH)) * sc_ecum[(tb * 16 + 4 * lq + r) >> rsl];
          } else {
            add_qh(acc);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[tb][r] *= sc_ecum[(tb * 16 + 4 * lq + r) >> rsl];
          }
          if (nb0 == 0) add_mx(acc);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) Yd[(tb * 16 + 4 * lq + r) * ys + p0 + l16] = acc[tb][r];
        } else {
          // One accumulator per 16-row block keeps independent MFMA chains in
          // flight; Q h'^T in its own accumulators, exp(cum) scales its rows
          // afterwards.
          floatx4 acc[TB], aci[TB];
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) {
            acc[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
            aci[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
          }
          if (nb0 == 0) add_mx(acc);
          add_qh(aci);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int v = tb * 16 + 4 * lq + r;
              Yd[v * ys + p0 + l16] = fmaf(sc_ecum[v >> rsl], aci[tb][r], acc[tb][r]);
            }
        }
      }
      // the next chunk's x rows land during the update and the epilogue (every
      // wave is an MFMA wave where they load late)
      if constexpr (LATE_X) {
        prefetch_x(c0 + Qt);
      }
      // ---- P5b: state update h' = decay h' + K^T (w X) ------------------------
      const float dec = run[64];
#pragma unroll
      for (int j = 0; j < (KT16 ? 0 : JMAX); ++j) Hacc[j] *= dec;
      if constexpr (SPLIT) {
        // B operand: w x of column p0 + l16 at virtual rows 4 lq + i, 16 + 4 lq + i
        float wx[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int v = 16 * (i >> 2) + 4 * lq + (i & 3);
          wx[i] = Xl[v * xs + p0 + l16] * sc_w[v >> rsl];
        }
        if constexpr (KT16) {
          // w x to fp16 head / tail, one scale per head_dim column; the
          // product of the two scales comes off each tile's three products
          float wm = 0.f;
#pragma unroll
          for (int i = 0; i < 8; i += 2) wm = max3_abs(wx[i], wx[i + 1], wm);
          const int eW = f16_scale_exp(max_xor16_32(wm));
          const float sW = ldexpf(1.f, eW);
          unsigned h0, h1, h2, h3, t0, t1, t2, t3;
          split2_f16s(wx[0], wx[1], sW, h0, t0);
          split2_f16s(wx[2], wx[3], sW, h1, t1);
          split2_f16s(wx[4], wx[5], sW, h2, t2);
          split2_f16s(wx[6], wx[7], sW, h3, t3);
          const uintx4 bh = uintx4{h0, h1, h2, h3}, bl = uintx4{t0, t1, t2, t3};
          const int esh = -(eK + eW);
#pragma unroll
          for (int j = 0; j < JMAX; ++j) {
            const int n = (nb0 + j) * 16 + l16;
            const int blk = 4 * (lq ^ ((n >> 2) & 3));
            const uintx4 ah = *reinterpret_cast<const uintx4*>(KTh + n * kKTw + blk);
            const uintx4 al = *reinterpret_cast<const uintx4*>(KTm + n * kKTw + blk);
            floatx4 d = mfma_f16(al, bh, floatx4{0.f, 0.f, 0.f, 0.f});
            d = mfma_f16(ah, bl, d);
            d = mfma_f16(ah, bh, d);
#pragma unroll
            for (int r = 0; r < 4; ++r) Hacc[j][r] = fmaf(Hacc[j][r], dec, ldexpf(d[r], esh));
          }
        } else {
          uintx4 bh, bm, bl;
          split8_bf16x3(wx, bh, bm, bl);
#pragma unroll
          for (int j = 0; j < JMAX; ++j) {
            const int n = (nb0 + j) * 16 + l16;
            const int blk = 4 * (lq ^ ((n >> 2) & 3));
            const uintx4 ah = *reinterpret_cast<const uintx4*>(KTh + n * kKTw + blk);
            const uintx4 am = *reinterpret_cast<const uintx4*>(KTm + n * kKTw + blk);
            const uintx4 al = *reinterpret_cast<const uintx4*>(KTl + n * kKTw + blk);
            Hacc[j] = mfma_bf16x6(ah, am, al, bh, bm, bl, Hacc[j]);
          }
        }
      }
      for (int sb = 0; sb < (SPLIT ? 0 : TB); ++sb) {
        const int v0 = sb * 16 + 4 * lq;
        const float* xc = Xl + v0 * xs + p0 + l16;
        const float xw0 = xc[0] * sc_w[(v0 + 0) >> rsl];
        const float xw1 = xc[xs] * sc_w[(v0 + 1) >> rsl];
        const float xw2 = xc[2 * xs] * sc_w[(v0 + 2) >> rsl];
        const float xw3 = xc[3 * xs] * sc_w[(v0 + 3) >> rsl];
        const float* kc = Kl + v0 * ks + nb0 * 16 + l16;
#pragma unroll
        for (int j = 0; j < JMAX; ++j) {
          if (FIXED || j < ntw) {
            Hacc[j] = mfma16(kc[j * 16], xw0, Hacc[j]);
            Hacc[j] = mfma16(kc[ks + j * 16], xw1, Hacc[j]);
            Hacc[j] = mfma16(kc[2 * ks + j * 16], xw2, Hacc[j]);
            Hacc[j] = mfma16(kc[3 * ks + j * 16], xw3, Hacc[j]);
          }
        }
      }
    }
    lds_barrier();

    // ---- P6: epilogue ---------------------------------------------------------
    if constexpr (FULL && !MIMO) {
      // out = (y + D x) * silu(z), VEC-wide and coalesced along head_dim
#pragma unroll
      for (int k = 0; k < KX; ++k) {
        const int idx = tid + k * nthreads;
        const int t = idx / xrow, pv = idx - t * xrow;
        // fixed-size variant: one item per thread, and rows past the chunk's
        // last token fall outside the store's buffer range, so the store
        // needs no branch (the compiler then counts it and the next
        // chunk's staging does not wait for it)
        if (FIXED || (idx < Qt * xrow && t < nvalid)) {
          vec_t y = vload<VEC>(Yl + t * ys + pv * VEC);
          if (NH > 1) y += vload<VEC>(Yl2 + t * ys + pv * VEC);
          const vec_t xv = vload<VEC>(Xl + t * xs + pv * VEC);
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            float v = comp(y, e);
            if (p.has_d) v = fmaf(dh, comp(xv, e), v);
            if (p.has_z) v *= silu_fast(comp(zr[k], e));
            set_comp(y, e, v);
          }
          bstore<VEC>(ores, (uint32_t)(t * tokx + pv * VEC), y);
        }
      }
      // the next chunk's raw maxima (its rows were prefetched before S;
      // this chunk's staging has read the slots)
      raw_maxima();
      lds_barrier();
    }
    if constexpr (FULL && MIMO) {
      // per rank: D skip, gate silu(z * mimo_z), optional RMS norm over P,
      // then the mimo_o-weighted sum over ranks; one wave per token
      const int pa = lane, pb = lane + 64;
#pragma unroll
      for (int i = 0; i < KZM; ++i) {
        const int t = wave + i * nwaves;
        if (t >= nvalid) break;  // wave-uniform
        float o0 = 0.f, o1 = 0.f;
        // ranks unrolled to the rank stride where it is known, so that their
        // norm reductions overlap
#pragma unroll
        for (int r = 0; r < (RSC > 0 ? RSC : R); ++r) {
          if (RSC > 0 && r >= R) break;  // uniform
          const int v = (t << rsl) + r;
          float y0 = 0.f, y1 = 0.f;
          if (pa < P) {
            y0 = Yl[v * ys + pa] + (NH > 1 ? Yl2[v * ys + pa] : 0.f);
            if (p.has_d) y0 = fmaf(dh, Xl[v * xs + pa], y0);
            if (p.has_z) y0 *= silu_fast(zm[i][0] * mzL[r * P + pa]);
          }
          if (pb < P) {
            y1 = Yl[v * ys + pb] + (NH > 1 ? Yl2[v * ys + pb] : 0.f);
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
        const uint32_t ob = (uint32_t)(t * tokx);
        if (pa < P) buf_store1(ores, (ob + pa) * 4u, o0);
        if (pb < P) buf_store1(ores, (ob + pb) * 4u, o1);
      }
      raw_maxima();  // the next chunk's (see the SISO epilogue)
      lds_barrier();
    }
  }

  if constexpr (!FULL) {
    const size_t si = (size_t)bh * nsum_all + seg;  // this piece
    float* st = p.ws_state + si * (size_t)(PT * NT) * 256;
    if (mma_wave) {
#pragma unroll
      for (int j = 0; j < JMAX; ++j)
        if (FIXED || j < ntw) *reinterpret_cast<floatx4*>(st + ((pt * NT + nb0 + j) * 64 + lane) * 4) = Hacc[j];
    }
    float* aux = p.ws_aux + si * kAux;
    if (tid < A) aux[tid] = run[tid];
    if (tid == (MERGED ? sw : 0) * 64) aux[kAuxDecay] = seg_decay;  // lane 0 of the scalar wave
  }
}

thread_local uint32_t g_forced_segments = 0;

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
  // at once (two per CU), so no CU runs a second round; each segment keeps at
  // least four chunks.
  const long target = 2L * device_cu_count();
  long nseg = 1;
  if (bhn < target) nseg = target / bhn;
  const long max_seg = ((long)g.L + 4L * Qt - 1) / (4L * Qt);
  if (nseg > max_seg) nseg = max_seg;
  // Segment s folds the summaries before it, so the fold's work grows with
  // the square of the segment count.  At most 65 segments keep the last
  // segment's fold within a few chunks' time where few chains would
  // otherwise ask for hundreds.
  if (nseg > kMaxAutoSegments) nseg = kMaxAutoSegments;
  if (g_forced_segments > 0) nseg = (long)g_forced_segments;
  if (nseg < 1) nseg = 1;
  long seg_len = ((long)g.L + nseg - 1) / nseg;
  seg_len = (seg_len + Qt - 1) / Qt * Qt;
  nseg = ((long)g.L + seg_len - 1) / seg_len;
  pl.nseg = (int)nseg;
  pl.seg_len = (int)seg_len;
  // With few segments the summary pass cuts each segment before the last
  // into two pieces of whole chunks: twice the workgroups over the same
  // tokens, where one summary per segment would leave CUs' second slots
  // idle (B4 H24: 384 workgroups; 768 in pieces ran the pass 4 us faster).
  // The main pass folds every earlier piece, so with many segments, or when
  // the pieces would take more than one and a half rounds of the slots, one
  // summary per segment is faster (the fold halves; B1 L65536 H32 / H4 / H1
  // 2% / 9% / 5% faster per call).
  pl.npc = (nseg > 1 && nseg <= 8 && 2L * bhn * (nseg - 1) <= 3L * device_cu_count()) ? 2 : 1;
  pl.plen = (int)(((seg_len / Qt + pl.npc - 1) / pl.npc) * Qt);
  const long nsum = (nseg - 1) * pl.npc;
  pl.ws_state_floats = nseg > 1 ? (size_t)bhn * nsum * PT * NT * 256 : 0;
  pl.ws_aux_floats = nseg > 1 ? (size_t)bhn * nsum * kAux : 0;
  return pl;
}

// LDS layout of one pass; the summary pass needs no Q, M or Y buffers.  Rows
// are padded by four floats so that rows 4 apart start 16 banks apart.
//
// With the split state update the keys are also kept split and transposed
// (o_kt: three bf16 planes in the summary pass, two fp16 planes in the main
// pass); the summary pass keeps no fp32 keys, and in the main pass the two raw
// y buffers overlay the fp32 keys (the fp16 query / key planes of the merged
// layout), whose last reader is S = Q K^T (a barrier separates it from the y
// writes); the key buffer is enlarged where the two do not fit in it.
void layout(ScanKParams& kp, bool full, bool mimo, bool split) {
  const int QV = kQV;
  kp.ks = kp.NT * 16 + 4;
  kp.xs = kp.PT * 16 + 4;
  kp.ms = QV + 4;
  kp.ys = kp.PT * 16 + 4;
  const bool y_over_k = full && split && kp.NH > 1;
  int off = 0;
  // the main pass of the split layout keeps Q and K as fp16 planes
  // [2][QV][kPQK] halves in these two regions
  const bool half = full && split;
  const int planes = half ? QV * kPQK : 0;  // floats of two fp16 planes
  kp.o_ql = off; off += full ? std::max(QV * kp.ks, planes) : 0;
  kp.o_kl = off;
  off += (full || !split) ? std::max(y_over_k ? std::max(QV * kp.ks, 2 * QV * kp.ys) : QV * kp.ks, planes) : 0;
  kp.o_kt = off; off += split ? (half ? 2 : 3) * kp.NT * 16 * kKTw : 0;  // main pass: two fp16 planes
  kp.o_xl = off; off += QV * kp.xs;
  kp.o_ml = off; off += full ? QV * kp.ms : 0;
  kp.o_ml2 = off; off += (full && kp.NH > 1) ? QV * kp.ms : 0;
  if (y_over_k) {
    kp.o_yl = kp.o_kl;
    kp.o_yl2 = kp.o_kl + QV * kp.ys;
  } else {
    kp.o_yl = off; off += full ? QV * kp.ys : 0;
    kp.o_yl2 = off; off += (full && kp.NH > 1) ? QV * kp.ys : 0;
  }
  // the entry-state fold overlays [PT*16][NT*16+4] floats on the chunk buffers,
  // or (the register fold, at most 128 summaries of 32 angles) three
  // [128][32] tables and 128 decays
  if (full && off < kp.PT * 16 * (kp.NT * 16 + 4)) off = kp.PT * 16 * (kp.NT * 16 + 4);
  if (full && off < 3 * 128 * 32 + 128) off = 3 * 128 * 32 + 128;
  kp.o_cs = off; off += 2 * 64;
  kp.o_bias = off; off += 2 * kp.R * kp.N;
  kp.o_mimo = off; off += mimo ? 3 * kp.R * kp.P + kp.P : 0;
  off = (off + 3) / 4 * 4;
  kp.o_sc = off; off += 6 * QV;
  kp.o_run = off; off += 72;
  kp.lds_floats = off;
}

// Raise a kernel's dynamic-LDS limit to one CU's 160 KiB, once per kernel and
// device (thread-safe; the attribute is set with that device current); later
// calls return the first call's status.
hipError_t set_max_lds_once(const void* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, hipError_t> done;
  std::lock_guard<std::mutex> lock(mu);
  auto it = done.find({dev, fn});
  if (it != done.end()) return it->second;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e != hipSuccess) (void)hipGetLastError();
  done.emplace(std::make_pair(dev, fn), e);
  return e;
}

// start / stop (optional): events the launch itself records around the
// kernel's execution (hipExtLaunchKernel), with no event commands of their
// own between the kernels in the stream
template <int VEC, bool FULL, bool MIMO, int NTC, int PTC, int NWC, int RSC, bool STR>
hipError_t launch_one(const ScanKParams& kp, unsigned grid, unsigned block, hipStream_t stream,
                      hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
  const size_t lds_bytes = (size_t)kp.lds_floats * sizeof(float);
  // Dynamic LDS above 64 KiB needs the opt-in attribute; set it once per
  // kernel instantiation to the largest layout it can take (the CU's 160 KiB)
  // and report a failure instead of launching.
  if (lds_bytes > 64 * 1024) {
    hipError_t e = set_max_lds_once(reinterpret_cast<const void*>(&scan_chunk_kernel<VEC, FULL, MIMO, NTC, PTC, NWC, RSC, STR>));
    if (e != hipSuccess) return e;
  }
  if (start != nullptr && stop != nullptr)
    hipExtLaunchKernelGGL((scan_chunk_kernel<VEC, FULL, MIMO, NTC, PTC, NWC, RSC, STR>), dim3(grid), dim3(block),
                          (std::uint32_t)lds_bytes, stream, start, stop, 0u, kp);
  else
    hipLaunchKernelGGL((scan_chunk_kernel<VEC, FULL, MIMO, NTC, PTC, NWC, RSC, STR>), dim3(grid), dim3(block), lds_bytes,
                       stream, kp);
  return hipGetLastError();
}

template <int VEC, bool MIMO, int NTC, int PTC, int NWC, int RSC, bool STR = false>
hipError_t launch_passes(ScanKParams kp, const ScanPlan& plan, unsigned bhn, unsigned block,
                         hipStream_t stream) {
  // as in the kernel: both passes of the merged layout run the split update
  constexpr bool kSplit = merged_variant(NTC, PTC, NWC, RSC);
  if (plan.nseg > 1) {
    ScanKParams ka = kp;
    layout(ka, false, MIMO, kSplit);
    hipError_t e = launch_one<VEC, false, MIMO, NTC, PTC, NWC, RSC, STR>(ka, bhn * (unsigned)((plan.nseg - 1) * plan.npc), block,
                                                                       stream);
    if (e != hipSuccess) return e;
  }
  layout(kp, true, MIMO, kSplit);
  const ProfileEvents& pe = profile_events();
  return launch_one<VEC, true, MIMO, NTC, PTC, NWC, RSC, STR>(kp, bhn * (unsigned)plan.nseg, block, stream, pe.start,
                                                              pe.stop);
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
  const bool strided = o.xs != 0 || o.ts != 0 || o.as != 0;
  if (strided && mimo) return hipErrorInvalidValue;  // packed rows feed the SISO scan only
  kp.NT = ((int)g.N + 15) / 16;
  kp.PT = ((int)g.P + 15) / 16;
  kp.NH = kp.NT > 4 ? 2 : 1;
  kp.NTH = (kp.NT + kp.NH - 1) / kp.NH;
  kp.RS = rank_stride((int)g.R);
  kp.rs_log2 = 0;
  while ((1 << kp.rs_log2) < kp.RS) ++kp.rs_log2;
  kp.Qt = kQV / kp.RS;
  kp.xstr = o.xs ? (int)o.xs : (int)(g.H * g.P);
  kp.tstr = o.ts ? (int)o.ts : (int)g.H;
  kp.astr = o.as ? (int)o.as : (int)g.A;
  kp.seg_len = plan.seg_len;
  kp.nseg = plan.nseg;
  kp.npc = plan.npc;
  kp.plen = plan.plen;
  float* ws = static_cast<float*>(workspace);
  kp.ws_state = ws;
  kp.ws_aux = ws ? ws + plan.ws_state_floats : nullptr;
  // 16-byte vector access needs every row width and row start on a 16-byte boundary.
  const bool vec4 = g.P % 4 == 0 && g.N % 4 == 0 && kp.xstr % 4 == 0 && aligned16(o.x) && aligned16(o.z) &&
                    aligned16(o.b) && aligned16(o.c) && aligned16(o.out);
  // One MFMA wave per (16 head_dim columns, N-part of at most four 16-wide
  // blocks); at least four waves; enough threads that every thread prefetches
  // at most KX x-vectors and KB B/C vectors (8P and 4N threads for both the
  // 16-byte and the scalar variant); and enough waves that the angle scan
  // (two angles per wave and pass, four passes) covers A.
  unsigned nwaves = (unsigned)(kp.PT * kp.NH);
  if (nwaves < 4u) nwaves = 4u;
  while (64u * nwaves < 8u * g.P) ++nwaves;
  while (64u * nwaves < 4u * g.N) ++nwaves;
  while (8u * nwaves < g.A) ++nwaves;
  const unsigned block = 64u * nwaves;
  const unsigned bhn = g.B * g.H;
  // The N = 128, P = 64 layers (eight waves) get a variant with compile-time
  // strides and rank stride; every other geometry runs the generic variant.
  if (vec4 && g.N == 128 && g.P == 64 && nwaves == 8 && g.A % 4 == 0 && kp.astr % 4 == 0 &&
      (g.A == 0 || aligned16(o.angle))) {
    if (!mimo)
      return strided ? launch_passes<4, false, 8, 4, 8, 1, true>(kp, plan, bhn, block, stream)
                     : launch_passes<4, false, 8, 4, 8, 1>(kp, plan, bhn, block, stream);
    switch (kp.RS) {
      case 1: return launch_passes<4, true, 8, 4, 8, 1>(kp, plan, bhn, block, stream);
      case 2: return launch_passes<4, true, 8, 4, 8, 2>(kp, plan, bhn, block, stream);
      case 4: return launch_passes<4, true, 8, 4, 8, 4>(kp, plan, bhn, block, stream);
      default: return launch_passes<4, true, 8, 4, 8, 8>(kp, plan, bhn, block, stream);
    }
  }
  if (strided)  // packed projection rows (SISO only)
    return vec4 ? launch_passes<4, false, 0, 0, 0, 0, true>(kp, plan, bhn, block, stream)
                : launch_passes<1, false, 0, 0, 0, 0, true>(kp, plan, bhn, block, stream);
  if (vec4)
    return mimo ? launch_passes<4, true, 0, 0, 0, 0>(kp, plan, bhn, block, stream)
                : launch_passes<4, false, 0, 0, 0, 0>(kp, plan, bhn, block, stream);
  return mimo ? launch_passes<1, true, 0, 0, 0, 0>(kp, plan, bhn, block, stream)
              : launch_passes<1, false, 0, 0, 0, 0>(kp, plan, bhn, block, stream);
}

}  // namespace

ProfileEvents& profile_events() {
  static thread_local ProfileEvents pe{nullptr, nullptr};
  return pe;
}

int device_cu_count() {
  constexpr int kMaxDev = 64;
  static std::once_flag once[kMaxDev];
  static int cus[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return 256;
  }
  std::call_once(once[dev], [dev] {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      v = 256;
    }
    cus[dev] = v;
  });
  return cus[dev];
}

void set_forced_segments(uint32_t nseg) { g_forced_segments = nseg; }

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
