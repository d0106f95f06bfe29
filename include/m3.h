/*
 * m3.h -- C ABI of the MI355X (gfx950) Mamba-3 selective-state path.
 *
 * Nine operations, named after the public functions of the oarust 0.8.6
 * source page src/rs/ml/matrix/mamba3.rs (its Public API section) and the
 * ml::matrix API index:
 *
 *   m3_preprocess   mamba3_preprocess   split + transform one packed projection
 *   m3_siso_fwd     mamba3_siso         SISO selective-state scan, forward
 *   m3_siso_fwd_packed  mamba3_preprocess + mamba3_siso, fused on the packed rows
 *   m3_mimo_fwd     mamba3_mimo         shared-state MIMO scan, forward
 *   m3_siso_step    mamba3_siso_step    one SISO decode token, states in place
 *   m3_mimo_step    mamba3_mimo_step    one MIMO decode token, states in place
 *   m3_siso_bwd     mamba3_siso_backward        the eleven SISO scan gradients
 *   m3_mimo_bwd     mamba3_mimo_backward        the fifteen MIMO scan gradients
 *   m3_preprocess_bwd mamba3_preprocess_backward gradients of projected, dt_bias
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers:   every tensor argument is a DEVICE pointer to contiguous,
 *             row-major float32 memory on the current HIP device, in exactly
 *             the layout the comment of that entry point gives.  Only the
 *             angle operands may be NULL, and only when num_rope_angles == 0
 *             (m3_preprocess_bwd also takes NULL for a missing gradient).
 * Ownership:  the caller allocates every input, output, state and workspace
 *             buffer.  The library allocates no device memory on these paths
 *             and keeps no pointer after the call returns.
 * Streams:    `stream` is a hipStream_t (NULL = the legacy default stream).
 *             All work is enqueued on it; no call synchronises the host.
 *             Outputs are valid once the stream reaches the call.
 * Errors:     each call returns an m3_status.  Geometry and shape rules are
 *             checked on the host before anything is enqueued, so on
 *             M3_ERR_INVALID_ARGUMENT or M3_ERR_UNSUPPORTED no device memory
 *             is touched (decode states stay as they were).  M3_ERR_HIP
 *             reports a failed kernel launch.  m3_last_error() returns a
 *             thread-local message naming the operation and the broken rule.
 * Threads:    calls are thread-safe; calls on different streams may overlap.
 * Precision:  float32 storage and arithmetic.  sin / cos are accurate to a
 *             few ulp; the state decay uses an accurate exp; the
 *             intra-chunk decay mask, exp(cum) and the SiLU gate use the
 *             hardware exp2 (relative error about |x| 2^-23).  At
 *             head_dim 64 / state 128 with 16-byte aligned operands the
 *             chunk state updates K^T (w x) (SISO: m3_siso_fwd,
 *             m3_siso_fwd_packed; MIMO: its segment summaries) take bf16
 *             matrix products of six-term splits (each fp32 operand as three
 *             bf16 pieces, six products accumulated in fp32): about 2^-23
 *             relative error per product, the fp32 level.
 */
#ifndef M3_H
#define M3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum m3_status {
    M3_OK = 0,
    M3_ERR_INVALID_ARGUMENT = 1, /* a geometry/shape rule of the operation is broken */
    M3_ERR_UNSUPPORTED = 2,      /* valid geometry beyond what the kernels implement */
    M3_ERR_HIP = 3               /* the HIP runtime rejected a launch */
} m3_status;

/*
 * Scan geometry and flags: mirror of the SsmConfig struct (mamba3.rs, Public
 * API section).  Passed by value.
 *   batch_size B, sequence_length L, num_heads H,
 *   num_groups G  (0 means G = H: one Q/K group per head),
 *   head_dim P, state_size N, num_rope_angles A (rotary pairs in the state
 *   axis), mimo_rank R (1 for SISO), and three 0/1 flags: has_z (SiLU z
 *   gate), has_d (D skip), has_output_norm (MIMO output RMS norm; SISO
 *   requires 0).
 * Head h reads B/C group g = h / (H / G).
 */
typedef struct m3_ssm_config {
    uint32_t batch_size;
    uint32_t sequence_length;
    uint32_t num_heads;
    uint32_t num_groups;
    uint32_t head_dim;
    uint32_t state_size;
    uint32_t num_rope_angles;
    uint32_t mimo_rank;
    uint32_t has_z;
    uint32_t has_d;
    uint32_t has_output_norm;
} m3_ssm_config;

/*
 * Preprocess geometry and bounds: mirror of the Mamba3PreprocessConfig struct
 * (mamba3.rs, Public API section).  inner_size I (width of the z and x slices),
 * state_size N, num_heads H, num_rope_angles A, num_groups G (>= 1 here),
 * mimo_rank R, RMS epsilon, inclusive dt bounds [dt_min, dt_max], and
 * a_floor, the positive floor of the A magnitude.
 */
typedef struct m3_preprocess_config {
    uint32_t inner_size;
    uint32_t state_size;
    uint32_t num_heads;
    uint32_t num_rope_angles;
    uint32_t num_groups;
    uint32_t mimo_rank;
    float epsilon;
    float dt_min;
    float dt_max;
    float a_floor;
} m3_preprocess_config;

/*
 * m3_preprocess -- mamba3_preprocess (PreprocessGeometry::resolve for the rules;
 * Mamba3PreprocessResult for the outputs).
 *
 * In:  projected [rows, W] with W = 2I + 2*G*R*N + 3H + A, columns in the
 *      order z | x | B | C | dt | A | trap | angle;  dt_bias [H].
 * Out: x, z [rows, I]  copies of their slices;
 *      bh, ch [rows, G*R*N]  each N-wide row v scaled by 1/sqrt(mean(v^2)+eps);
 *      dt [rows, H]   = clamp(softplus(dt_raw + dt_bias[h]), dt_min, dt_max);
 *      adt [rows, H]  = -max(softplus(A_raw), a_floor) * dt;
 *      trap [rows, H], angle [rows, A]  copies (raw gate, raw angular velocity).
 * Rules (M3_ERR_INVALID_ARGUMENT): rows, I, N, H, G, R > 0; 2A <= N;
 *      epsilon, dt_min, dt_max, a_floor finite; epsilon, dt_min, a_floor > 0;
 *      dt_min <= dt_max; every element count and W fit in uint32.
 * `angle` may be NULL when A == 0.  Outputs must not alias the inputs.
 */
int m3_preprocess(const float* projected, const float* dt_bias, uint32_t rows,
                  m3_preprocess_config cfg,
                  float* x, float* z, float* bh, float* ch,
                  float* dt, float* adt, float* trap, float* angle,
                  void* stream);

/*
 * m3_siso_fwd -- mamba3_siso (Geometry::resolve for the rules).  Operands in
 * the pages' order, C before B:
 *   c, b [B,L,G,N];  x, z [B,L,H,P];  adt, dt, trap [B,L,H];  angle [B,L,A];
 *   c_bias, b_bias [H,N];  d [H]   ->   out [B,L,H,P].
 * Per (batch, head), from a zero state, for t = 0..L-1:
 *   theta_t = theta_{t-1} + dt_t * angle_t;  lam_t = sigmoid(trap_t);
 *   K_t = rot(B_t + b_bias, theta_t);  Q_t = rot(C_t + c_bias, theta_t);
 *   h_t = e^{adt_t} h_{t-1} + (1-lam_t) dt_t e^{adt_t} x_{t-1} K_{t-1}^T
 *         + lam_t dt_t x_t K_t^T;
 *   out_t = (h_t Q_t + has_d * D x_t) * (has_z ? silu(z_t) : 1)
 * where rot() turns split-half pairs (a, a+A) of the state axis by theta_a.
 * z and d are read only when their flag is set but must be valid pointers.
 * Rules (M3_ERR_INVALID_ARGUMENT): B, L, H, G, P, N > 0; H % G == 0;
 *   P <= 128; N <= 128; A <= 64; 2A <= N; mimo_rank == 1;
 *   has_output_norm == 0; flags 0 or 1; element counts and B*H fit uint32.
 * workspace: at least m3_siso_fwd_workspace_bytes(cfg) bytes of device
 *   memory (may be NULL when that is 0); its contents on entry are ignored.
 * `out` must not alias any input.
 */
size_t m3_siso_fwd_workspace_bytes(m3_ssm_config cfg);
int m3_siso_fwd(const float* c, const float* b, const float* x, const float* z,
                const float* adt, const float* dt, const float* trap, const float* angle,
                const float* c_bias, const float* b_bias, const float* d,
                m3_ssm_config cfg, float* out,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * m3_siso_fwd_noalloc -- m3_siso_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same operands, layouts, rules and
 * result as m3_siso_fwd (the same kernels run), but no workspace argument:
 * the segment summaries go to a fixed 64 MiB scratch array in device memory
 * that the library holds on every GPU it runs on until the process ends.
 * The call allocates nothing.  Returns M3_ERR_UNSUPPORTED when
 * m3_siso_fwd_workspace_bytes(cfg) exceeds 64 MiB (not reached at
 * head_dim 64 / state_size 128 for any batch, heads or length).  Every call
 * on one GPU shares that GPU's scratch: calls that overlap on one GPU (two
 * streams, two threads) race and must be ordered by the caller.  The
 * scratch needs no clearing: each call writes every part it reads.
 */
int m3_siso_fwd_noalloc(const float* c, const float* b, const float* x, const float* z,
                        const float* adt, const float* dt, const float* trap, const float* angle,
                        const float* c_bias, const float* b_bias, const float* d,
                        m3_ssm_config cfg, float* out, void* stream);

/*
 * m3_siso_fwd_packed -- mamba3_preprocess followed by mamba3_siso in one
 * call that reads the packed projection rows directly.  projected [B*L, W]
 * (W = 2I + 2GN + 3H + A, columns z | x | B | C | dt | A | trap | angle) and
 * dt_bias [H] as for m3_preprocess; c_bias, b_bias [H,N] and d [H] as for
 * m3_siso_fwd; out [B,L,H,P].  out equals m3_siso_fwd applied to the eight
 * outputs of m3_preprocess of the same rows, but x, z, trap and angle are
 * read in place from the packed rows instead of being copied out, and only
 * the normalised B/C rows and dt / adt go through the workspace.  When W,
 * I and the angle column offset 2I + 2GN + 3H are multiples of 4 (16-byte
 * rows, as the dense operands have), the same kernel variant runs and the
 * result is identical bit for bit; otherwise a scalar-load variant runs
 * and may sum in another order (differences at float32 rounding level).
 * workspace: at least m3_siso_fwd_packed_workspace_bytes(pcfg, cfg) bytes
 *   (B*L*(2GN + 2H) floats plus the scan's own workspace); required.
 * Rules: those of m3_preprocess (rows = B*L) and of m3_siso_fwd, and the two
 *   configs must agree: inner_size == H*P, state_size == N, num_heads == H,
 *   num_rope_angles == A, num_groups == G (after G = 0 resolves to H),
 *   mimo_rank == 1 (M3_ERR_INVALID_ARGUMENT otherwise).
 */
size_t m3_siso_fwd_packed_workspace_bytes(m3_preprocess_config pcfg, m3_ssm_config cfg);
int m3_siso_fwd_packed(const float* projected, const float* dt_bias, const float* c_bias,
                       const float* b_bias, const float* d, m3_preprocess_config pcfg,
                       m3_ssm_config cfg, float* out, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * m3_mimo_fwd -- mamba3_mimo (MimoGeometry::resolve for the rules).  Operands:
 *   c, b [B,L,R*G,N] (row r*G + g is rank r of group g);  x, z [B,L,H,P];
 *   adt, dt, trap [B,L,H];  angle [B,L,A];  c_bias, b_bias [H,R,N];  d [H];
 *   mimo_x, mimo_z, mimo_o [H,R,P];  norm_weight [H,P]  ->  out [B,L,H,P].
 * One state per (batch, head) fed by every rank: with X_r = x * mimo_x[h,r]
 * and K_r, Q_r as in m3_siso_fwd from row r*G+g and biases [h,r],
 *   h_t = e^{adt_t} h_{t-1} + (1-lam_t) dt_t e^{adt_t} sum_r X_r,{t-1} K_r,{t-1}^T
 *         + lam_t dt_t sum_r X_r,t K_r,t^T;
 *   Y_r = (h_t Q_r,t + has_d * D X_r,t) * (has_z ? silu(z_t * mimo_z[h,r]) : 1);
 *   if has_output_norm: Y_r = Y_r / sqrt(mean_p(Y_r^2) + 1e-5) * norm_weight[h];
 *   out_t = sum_r mimo_o[h,r] * Y_r.
 * norm_weight is read only when has_output_norm == 1 but must be valid.
 * Rules: as m3_siso_fwd with 1 <= mimo_rank <= 8 and has_output_norm 0/1.
 *   The pages' cap P*N <= 4096 is a capacity limit of their kernel and is
 *   not applied: P, N <= 128 each.
 * workspace: at least m3_mimo_fwd_workspace_bytes(cfg) bytes (NULL if 0).
 */
size_t m3_mimo_fwd_workspace_bytes(m3_ssm_config cfg);
int m3_mimo_fwd(const float* c, const float* b, const float* x, const float* z,
                const float* adt, const float* dt, const float* trap, const float* angle,
                const float* c_bias, const float* b_bias, const float* d,
                const float* mimo_x, const float* mimo_z, const float* mimo_o,
                const float* norm_weight,
                m3_ssm_config cfg, float* out,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * m3_siso_step -- mamba3_siso_step (dispatch_mamba3_siso_step for the
 * state shapes).  The eleven operands take their L == 1 shapes
 * (c, b [B,1,G,N]; x, z [B,1,H,P]; adt, dt, trap [B,1,H]; angle [B,1,A];
 * biases [H,N]; d [H]).  States, read and written in place:
 *   ssm_state   [B,H,P,N]  h
 *   angle_state [B,H,A]    cumulative angle theta
 *   k_state     [B,H,N]    previous key (rotated, bias added)
 *   v_state     [B,H,P]    previous value (the previous token's x)
 * One token of the m3_siso_fwd recurrence, continuing from these states;
 * afterwards angle_state = theta_t, k_state = K_t, v_state = x_t.  A
 * sequence of L steps from zero states equals m3_siso_fwd over L tokens.
 * Rules: as m3_siso_fwd plus sequence_length == 1.  States are modified
 * only by a call that returns M3_OK.  States must not alias each other or
 * the operands; out [B,1,H,P] must not alias anything.
 */
int m3_siso_step(const float* c, const float* b, const float* x, const float* z,
                 const float* adt, const float* dt, const float* trap, const float* angle,
                 const float* c_bias, const float* b_bias, const float* d,
                 float* ssm_state, float* angle_state, float* k_state, float* v_state,
                 m3_ssm_config cfg, float* out, void* stream);

/*
 * m3_mimo_step -- mamba3_mimo_step (dispatch_mamba3_mimo_step for the state shapes).  The fifteen operands of
 * m3_mimo_fwd take their L == 1 shapes (c, b [B,1,R*G,N]; x, z [B,1,H,P];
 * adt, dt, trap [B,1,H]; angle [B,1,A]; biases [H,R,N]; d [H];
 * mimo_x, mimo_z, mimo_o [H,R,P]; norm_weight [H,P]).  States, read and
 * written in place:
 *   ssm_state   [B,H,P,N]    h (one state per head, fed by every rank)
 *   angle_state [B,H,A]      cumulative angle theta
 *   k_state     [B,H,R,N]    previous key of each rank (rotated, bias added)
 *   v_state     [B,H,R,P]    previous value of each rank (x * mimo_x[h,r])
 * One token of the m3_mimo_fwd recurrence, continuing from these states;
 * afterwards angle_state = theta_t, k_state[r] = K_r,t, v_state[r] = X_r,t.
 * A sequence of L steps from zero states equals m3_mimo_fwd over L tokens.
 * Rules: as m3_mimo_fwd plus sequence_length == 1.  States are modified
 * only by a call that returns M3_OK.  States must not alias each other or
 * the operands; out [B,1,H,P] must not alias anything.
 */
int m3_mimo_step(const float* c, const float* b, const float* x, const float* z,
                 const float* adt, const float* dt, const float* trap, const float* angle,
                 const float* c_bias, const float* b_bias, const float* d,
                 const float* mimo_x, const float* mimo_z, const float* mimo_o,
                 const float* norm_weight,
                 float* ssm_state, float* angle_state, float* k_state, float* v_state,
                 m3_ssm_config cfg, float* out, void* stream);

/*
 * m3_siso_bwd -- mamba3_siso_backward (SsmBackward for the eleven
 * gradients).  Given the upstream
 * gradient dout [B,L,H,P] of m3_siso_fwd's output and the same eleven
 * operands and config as the forward call, writes the gradient of
 * sum(dout * out) with respect to every operand, each in its operand's
 * layout:
 *   d_c, d_b [B,L,G,N] (summed over the heads of each group);
 *   d_x, d_z [B,L,H,P];  d_adt, d_dt, d_trap [B,L,H];  d_angle [B,L,A]
 *   (summed over heads);  d_c_bias, d_b_bias [H,N] and d_d [H] (summed over
 *   batch and sequence).
 * d_z is all zeros when has_z == 0 and d_d all zeros when has_d == 0.
 * Outputs are overwritten, not accumulated; they must not alias inputs.
 * workspace: at least m3_siso_bwd_workspace_bytes(cfg) bytes of device
 *   memory (chunk-entry states and exit adjoints [B*H, ceil(L/32), P, N]
 *   twice, per-head query/key adjoints [B,L,H,N] twice, and small
 *   per-token arrays); the contents need no initialisation.
 * Rules: those of m3_siso_fwd (M3_ERR_INVALID_ARGUMENT), plus
 *   M3_ERR_UNSUPPORTED when the group reduction's tile of 2 * (H/G) * N
 *   bias sums (plus a few rows) exceeds one CU's 160 KiB of LDS, which takes
 *   more than about 150 heads per group at N = 128.  d_angle may be NULL
 *   when A == 0.  The reductions run in a fixed order, so repeated calls
 *   with the same pointers give identical results.  At N = 128, P = 64,
 *   A = 32, kernels compiled for that geometry run when b, c, x, z, dout,
 *   both biases and the workspace are 16-byte aligned; with a misaligned
 *   one the general kernels run, whose results may differ in the last bits.
 */
size_t m3_siso_bwd_workspace_bytes(m3_ssm_config cfg);
int m3_siso_bwd(const float* dout, const float* c, const float* b, const float* x,
                const float* z, const float* adt, const float* dt, const float* trap,
                const float* angle, const float* c_bias, const float* b_bias, const float* d,
                m3_ssm_config cfg,
                float* d_c, float* d_b, float* d_x, float* d_z, float* d_adt, float* d_dt,
                float* d_trap, float* d_angle, float* d_c_bias, float* d_b_bias, float* d_d,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * m3_mimo_bwd -- mamba3_mimo_backward (Mamba3MimoBackward for the fifteen
 * gradients).  Given dout [B,L,H,P] and the fifteen
 * operands and config of the m3_mimo_fwd call, writes the gradient of
 * sum(dout * out) for every operand in its layout: d_c, d_b [B,L,R*G,N]
 * (row r*G + g, summed over the group's heads); d_x, d_z [B,L,H,P];
 * d_adt, d_dt, d_trap [B,L,H]; d_angle [B,L,A]; d_c_bias, d_b_bias [H,R,N];
 * d_d [H]; d_mimo_x, d_mimo_z, d_mimo_o [H,R,P]; d_norm_weight [H,P]
 * (all zeros without the norm; d_z and d_mimo_z zero without the gate,
 * d_d zero without the skip).  Outputs are overwritten.
 * workspace: at least m3_mimo_bwd_workspace_bytes(cfg) bytes.  Chunks hold
 *   32 / RS tokens (RS = R rounded up to a power of two), and the entry
 *   states and exit adjoints [B*H, chunks, P, N] dominate: 8.6 GB at
 *   B8 L4096 H32 P64 N128 R4.
 * Rules: those of m3_mimo_fwd, plus M3_ERR_UNSUPPORTED when a kernel's
 *   working set exceeds one CU's 160 KiB of LDS.  Fixed-order reductions:
 *   repeated calls with the same pointers give identical results.  As for
 *   m3_siso_bwd, N = 128 / P = 64 / A = 32 with 16-byte aligned operands
 *   (mimo_x included) and workspace takes kernels compiled for that
 *   geometry, which may differ from the general ones in the last bits.
 */
size_t m3_mimo_bwd_workspace_bytes(m3_ssm_config cfg);
int m3_mimo_bwd(const float* dout, const float* c, const float* b, const float* x,
                const float* z, const float* adt, const float* dt, const float* trap,
                const float* angle, const float* c_bias, const float* b_bias, const float* d,
                const float* mimo_x, const float* mimo_z, const float* mimo_o,
                const float* norm_weight, m3_ssm_config cfg,
                float* d_c, float* d_b, float* d_x, float* d_z, float* d_adt, float* d_dt,
                float* d_trap, float* d_angle, float* d_c_bias, float* d_b_bias, float* d_d,
                float* d_mimo_x, float* d_mimo_z, float* d_mimo_o, float* d_norm_weight,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * m3_preprocess_bwd -- mamba3_preprocess_backward (gradients of projected
 * and dt_bias; Mamba3PreprocessBackward).  projected [rows, W], dt_bias [H]
 * and cfg as for m3_preprocess; g_x, g_z [rows, I], g_bh, g_ch
 * [rows, G*R*N], g_dt, g_adt, g_trap [rows, H], g_angle [rows, A] are the
 * gradients of the eight preprocess outputs, and any of them may be NULL,
 * which counts as a zero gradient.  Writes d_projected [rows, W]:
 *   z, x, trap, angle columns: the output gradient;
 *   B, C columns, per N-wide row v with y = v / sqrt(mean(v^2) + eps):
 *     r * g - v * r^3 * mean(g * v),  r = 1 / sqrt(mean(v^2) + eps);
 *   dt columns: (g_dt - max(softplus(A_raw), a_floor) * g_adt) * sigmoid(u),
 *     u = dt_raw + dt_bias, where dt_min <= softplus(u) <= dt_max, else 0;
 *   A columns: -dt * g_adt * sigmoid(A_raw) where softplus(A_raw) >= a_floor,
 *     else 0;
 * and d_dt_bias [H] = the column sums of the dt columns, in a fixed order.
 * Rules: those of m3_preprocess.
 */
int m3_preprocess_bwd(const float* projected, const float* dt_bias, uint32_t rows,
                      m3_preprocess_config cfg,
                      const float* g_x, const float* g_z, const float* g_bh, const float* g_ch,
                      const float* g_dt, const float* g_adt, const float* g_trap,
                      const float* g_angle, float* d_projected, float* d_dt_bias, void* stream);

/*
 * Measurement hook.  After m3_set_profile_events(start, stop) with two
 * hipEvent_t handles, later m3_siso_fwd / m3_siso_fwd_packed / m3_mimo_fwd
 * calls on this thread launch their main scan kernel with the two events
 * attached (hipExtLaunchKernelGGL): `start` is recorded as the kernel
 * begins and `stop` as it ends, on the call's stream, so
 * hipEventElapsedTime(start, stop) is that kernel's duration with no event
 * command of its own in the stream.  Both handles must be non-NULL; a NULL
 * in either turns the hook off.  The caller owns the events.
 */
void m3_set_profile_events(void* start_event, void* stop_event);

/*
 * Scan plan override (testing and tuning).  The scan cuts each sequence
 * into segments that run in parallel, after a first pass that summarises
 * every segment but the last; by default the count fills two workgroups per
 * compute unit of the current device.  m3_set_scan_segments(n) with n > 0
 * makes later m3_siso_fwd, m3_siso_fwd_packed and m3_mimo_fwd calls (and
 * their workspace queries) on this thread use n segments, fewer when the
 * sequence has fewer whole chunks; n = 0 restores the default.  Results
 * agree to float32 rounding whatever the count.
 */
void m3_set_scan_segments(uint32_t segments);

/* Thread-local message of the last failed call on this thread (empty if none). */
const char* m3_last_error(void);

/* Library version string. */
const char* m3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* M3_H */
