/*
 * ssd.h - C ABI of the MI355X (gfx950) Mamba-2 SSD chunked forward.
 *
 * Two paths compute the SSD block's forward pass as a chunked selective scan:
 *   SSD_PATH_FLOAT  floating-point chunk algebra (fp16/bf16 MFMA, fp32 accumulate)
 *   SSD_PATH_INT8   the persistent-INT8 path of "SSDi8: Accurate and Efficient
 *                   8-bit Quantization for State Space Duality" (paper notes page,
 *                   ICLR 2026), sections "Overall framework" and "Key designs 1-3".
 *
 * The operation (the selective state-space recurrence the SSDi8 "Overall
 * framework" splits into chunks L = c*l; zero initial state):
 *   h_t[h,p,n] = exp(dt_t[h] A[h]) h_{t-1}[h,p,n] + dt_t[h] x_t[h,p] B_t[g(h),n]
 *   y_t[h,p]   = sum_n C_t[g(h),n] h_t[h,p,n] + D[h] x_t[h,p]
 * with head h in group g(h) = h / (H/G).
 *
 * Layouts (row-major, contiguous, no strides):
 *   X, Y   [B, L, H, P]     dt [B, L, H]     B, C [B, L, G, N]     A, D [H] fp32
 *   qB, qC [B, L, G, N] int8
 *   dAcs, lut [B, H, c, l] fp32            qdecay [B, H, c] uint8
 *   states [B, c, H, P, N]  int8 (INT8 path) or fp32 (float path)
 *   CB     [B, c, G, l, l]  int32 (INT8 path) or fp32 (float path)
 *   final_state [B, H, P, N] int8 or fp32
 * where c = ceil(L / l). A partial last chunk behaves as if zero padded
 * (dt = 0 steps leave the state unchanged); padded positions of dAcs hold the
 * last valid cumulative value and of lut hold 0.
 *
 * Ownership: every buffer is allocated by the caller in device memory (except
 * the shape, scale and tap descriptors, which are host structs holding device
 * pointers) and must be 16-byte aligned (the scale arrays: 4-byte aligned).
 * The library never allocates, frees or keeps a caller's pointer after a call
 * returns, and may be called from several threads on different streams. Its
 * only global state belongs to ssd_forward_noalloc: one fixed device array per
 * device and a mutex-guarded table of their addresses.
 *
 * Streams: `stream` is a hipStream_t (NULL = the null stream). Calls only
 * enqueue work; results are valid once the stream has been synchronised.
 *
 * Errors: every call validates all arguments before enqueueing anything; a
 * call that returns an error has written nothing. No C++ exception crosses
 * this interface. Preconditions that are NOT checked: finite inputs, dt > 0,
 * A < 0 (so every decay is <= 1), finite positive scales, and that output
 * buffers do not overlap inputs (except where a call says "in place").
 */
#ifndef MAMBA_SSD_CHUNKED_AMD_SSD_H
#define MAMBA_SSD_CHUNKED_AMD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-valued call. */
enum {
  SSD_OK = 0,
  SSD_E_NULL = 1,        /* a required pointer is NULL */
  SSD_E_SHAPE = 2,       /* negative or zero sizes, H % G != 0, size overflow */
  SSD_E_UNSUPPORTED = 3, /* chunk not in {64,128,256}, P not in {16,32,64},
                            N not in {16,32,64,128}, unknown dtype or path */
  SSD_E_ALIGN = 4,       /* a buffer is not 16-byte aligned */
  SSD_E_WORKSPACE = 5,   /* workspace smaller than ssd_workspace_bytes() */
  SSD_E_HIP = 6,         /* the HIP runtime reported a launch error */
  SSD_E_INTERNAL = 7,
  SSD_E_VALUE = 8,       /* a calibration maximum is negative, NaN or infinite */
  SSD_E_TOO_LARGE = 9    /* ssd_forward_noalloc: the problem needs more workspace
                            than SSD_NOALLOC_SCRATCH_BYTES */
};

/* Element type of X, dt, B, C and Y. */
enum { SSD_DTYPE_F32 = 0, SSD_DTYPE_F16 = 1, SSD_DTYPE_BF16 = 2 };

/* Which path a call computes. The two ablation rows of the notes page's
 * Table 5 (experiments: the latency ladder from the float SSD to the full
 * method) are ssd_forward paths only:
 *   SSD_PATH_ABL_QX     "+ Q(X) only": X quantised once per (h,p) with its own
 *                       static step (scales s_Xq, inv_Xq), everything else the
 *                       float path on Q(X) s_Xq; the state stays fp32.
 *   SSD_PATH_ABL_RECON  "+ reconstruction + B,C quantisation": Q(B), Q(C) once;
 *                       ChunkState on INT8 through the reconstruction
 *                       (S32 = Q(X_scaled) x Q(B)), dequantised with s_X s_B and
 *                       passed in fp32; ChunkScan1 on INT8 (the passed state
 *                       quantised with s_S, Q(C)); ChunkBMM and ChunkScan2 in
 *                       floating point on B and C. */
enum { SSD_PATH_FLOAT = 0, SSD_PATH_INT8 = 1, SSD_PATH_ABL_QX = 2, SSD_PATH_ABL_RECON = 3 };

/* Problem shape. batch == 0 or seqlen == 0 is a valid empty problem: calls
 * return SSD_OK and enqueue nothing, except that with seqlen == 0 and batch > 0
 * ssd_forward and ssd_state_passing write final_state (when given) as the state
 * after no positions: a copy of initial_state, or zeros without one. Every
 * other size must be > 0. */
typedef struct ssd_shape {
  int64_t batch;    /* B */
  int64_t seqlen;   /* L */
  int64_t nheads;   /* H */
  int64_t headdim;  /* P */
  int64_t dstate;   /* N */
  int64_t ngroups;  /* G, divides H */
  int64_t chunk;    /* l */
  int32_t dtype;    /* SSD_DTYPE_* */
  int32_t schedule; /* SSD_SCHED_*: 0 (auto) unless a schedule is wanted */
} ssd_shape;

/* Work schedule of ssd_forward on SSD_PATH_INT8 with fp16 or bf16 inputs
 * (other calls, paths and dtypes accept any of these values and ignore it;
 * any other value returns SSD_E_SHAPE):
 *   SSD_SCHED_HEAD   one persistent workgroup per head walks its chunks in
 *                    order, the state kept on chip (fewest HBM bytes);
 *   SSD_SCHED_CHUNK  ChunkState for every chunk in parallel, StatePassing,
 *                    then ChunkScan for every chunk in parallel (more bytes,
 *                    but B * c * H workgroups fill the GPU when B * H heads
 *                    cannot);
 *   SSD_SCHED_AUTO   SSD_SCHED_CHUNK when B * H is below twice the device's
 *                    compute-unit count, SSD_SCHED_HEAD otherwise.
 * Both give the same integers (taps, final state) and Y to within fp32
 * rounding order; ssd_workspace_bytes depends on the schedule. */
enum { SSD_SCHED_AUTO = 0, SSD_SCHED_HEAD = 1, SSD_SCHED_CHUNK = 2 };

/* Static scale pack of the INT8 path (device fp32 arrays). Step sizes
 * s = amax / 127 ("Key design 2" and "Training strategy": static symmetric
 * scales; B/C per group G, X_scaled and the state per (H,P)).
 *   s_B, s_C, inv_B, inv_C   [G]       inv = fp32(1 / s)
 *   inv_X, s_S, M_req        [H * P]   M_req = fp32(s_X * s_B[g(h)] / s_S)
 * The ablation paths read more (each may be NULL where no path reads it):
 *   s_X                      [H * P]   X_scaled step (SSD_PATH_ABL_RECON)
 *   s_Xq, inv_Xq             [H * P]   step of X itself (SSD_PATH_ABL_QX only;
 *                                      that path reads no other array)
 */
typedef struct ssd_scales {
  const float* s_B;
  const float* s_C;
  const float* inv_B;
  const float* inv_C;
  const float* inv_X;
  const float* s_S;
  const float* M_req;
  const float* s_X;
  const float* s_Xq;
  const float* inv_Xq;
} ssd_scales;

/* Optional debug outputs of the INT8 path (any member may be NULL). */
typedef struct ssd_taps {
  int8_t* q_xs;      /* Q(X_scaled)            [B, L, H, P] */
  int32_t* s32;      /* State_INT32 per chunk  [B, c, H, P, N] */
  int8_t* s8_local;  /* State_INT8 per chunk before StatePassing [B, c, H, P, N] */
  int8_t* passed;    /* states after StatePassing [B, c, H, P, N] (ssd_forward only) */
} ssd_taps;

/* ChunkBMM/ChunkScan B/C input quantisation, once per group ("Overall
 * framework": B and C are quantised along G once at SSD entry and reused;
 * "Key design 3").  qB = sat127(RHAZ(fl32(fl32(B) * inv_B[g]))), same for C,
 * with round-half-away-from-zero and single float32 roundings.
 * B, C: [B,L,G,N] in shape->dtype. scales: inv_B, inv_C used. */
int ssd_quantize_bc(const ssd_shape* shape, const void* B, const void* C,
                    const ssd_scales* scales, int8_t* qB, int8_t* qC, void* stream);

/* ChunkCumsum ("Overall framework": kept in floating point).
 * Per (b, h, chunk k): a_s = sum_{s'<=s} dt_s' * A[h], accumulated in float64
 * in sequence order. Writes dAcs = fp32(a_s); lut = fp32(dt_s * exp(a_{l-1} - a_s))
 * evaluated in float64 (LUT_state of "Key design 1", Eq. 4); and, if qdecay is
 * not NULL, qdecay = min(128, RHAZ(128 * exp(a_{l-1}))) decided in float64
 * (the fixed-point Decay of "Key design 2", Eq. 6, S = 2^7).
 * lut and qdecay may be NULL. */
int ssd_chunk_cumsum(const ssd_shape* shape, const void* dt, const float* A, float* dAcs,
                     float* lut, uint8_t* qdecay, void* stream);

/* ChunkState ("Key design 1": State = X x (B . LUT_state), Eq. 4, computed as
 * the reconstruction Q(X_scaled) x Q(B)).
 * INT8: Q(Xs)[t,h,p] = sat127(RHAZ(fl32(fl32(lut * x) * inv_X[h,p]))),
 *       S32 = sum_s Q(Xs)[s,h,p] Q(B)[s,g,n] (int8 MFMA, int32 accumulate),
 *       states = sat127(RHAZ(fl32(fl32(S32) * M_req[h,p]))) (requantised in
 *       registers, "Key design 2"). Bq = qB (int8); states int8; taps optional.
 * FLOAT: states[k,h,p,n] = sum_s lut_s x[s,h,p] B[s,g,n] in fp32 (MFMA on
 *       operands in the input dtype); Bq = B in shape->dtype; states fp32;
 *       scales and taps are ignored and may be NULL. */
int ssd_chunk_state(const ssd_shape* shape, int path, const void* X, const float* lut,
                    const void* Bq, const ssd_scales* scales, void* states,
                    const ssd_taps* taps, void* stream);

/* StatePassing (Eq. 6 of "Key design 2"), in place over `states`, sequential
 * over chunks. INT8: H_0 = S_0, H_k = sat127(S_k + RSH7(qdecay_k * H_{k-1}))
 * with RSH7(v) = sign(v) * ((|v| + 64) >> 7); qdecay required, dAcs unused.
 * FLOAT: H_k = exp(dAcs[k, l-1]) * H_{k-1} + S_k in fp32; qdecay unused.
 * initial_state (may be NULL): the state before chunk 0, [B,H,P,N], int8 in
 * the state scale s_S (INT8) or fp32 (FLOAT); when given, the update applies
 * from k = 0 with H_{-1} = initial_state (a previous call's final_state
 * continues that sequence).
 * On return slot k holds H_k (the state after chunk k). final_state (may be
 * NULL) receives H_{c-1}. */
int ssd_state_passing(const ssd_shape* shape, int path, void* states, const float* dAcs,
                      const uint8_t* qdecay, const void* initial_state, void* final_state,
                      void* stream);

/* ChunkBMM ("Key design 2": reuses the INT8 B and C):
 * CB[b,k,g,i,j] = sum_n Cq[k*l+i, g, n] * Bq[k*l+j, g, n] for j <= i, 0 above
 * the diagonal. INT8: Cq, Bq int8, CB int32 (exact). FLOAT: input dtype,
 * CB fp32. Positions past L contribute 0. */
int ssd_chunk_bmm(const ssd_shape* shape, int path, const void* Cq, const void* Bq,
                  void* CB, void* stream);

/* ChunkScan1 + ChunkScan2 + the D skip ("Key design 2").
 *   Scan1 (k >= 1): Y_off[s,p] = exp(dAcs_s) * sum_n C[s,n] H_{k-1}[p,n]; on the
 *     INT8 path C = Q(C), H = int8 states and the sum is dequantised with
 *     s_C[g] * s_S[h,p].
 *   Scan2: Y_diag[s,p] = sum_{s'<=s} CB[s,s'] exp(dAcs_s - dAcs_s') dt_s' x[s',p]
 *     (INT8: CB int32 with its dequant s_C * s_B folded into the LUT).
 *   Y = Y_off + Y_diag + D[h] x, stored in shape->dtype.
 * states are the passed states (slot k-1 feeds chunk k); initial_state (may
 * be NULL, same type and layout as in ssd_state_passing) feeds chunk 0. */
int ssd_chunk_scan(const ssd_shape* shape, int path, const void* X, const void* dt,
                   const float* dAcs, const void* Cq, const void* CB, const void* states,
                   const void* initial_state, const float* D, const ssd_scales* scales, void* Y,
                   void* stream);

/* The whole SSD forward in one call ("Overall framework": all modules).
 * B, C, X, dt in shape->dtype; Y in shape->dtype. INT8 needs scales.
 * path may also be one of the two ablation rows (SSD_PATH_ABL_QX,
 * SSD_PATH_ABL_RECON: module kernels, fp32 final_state, no initial_state and
 * no taps; an initial_state returns SSD_E_UNSUPPORTED).
 * initial_state (may be NULL): the state before the first position, int8 in
 * the state scale (INT8) or fp32 (FLOAT) [B,H,P,N]; passing a previous call's
 * final_state continues that sequence (exactly, when the previous call's
 * length was a multiple of the chunk size).
 * final_state (may be NULL): int8 (INT8) or fp32 (FLOAT) [B,H,P,N].
 * workspace: device memory of at least ssd_workspace_bytes(shape, path) bytes
 * (may be NULL when that is 0). taps: INT8 only, may be NULL. The integer
 * intermediates are bit-identical to those of the module calls above. */
int ssd_forward(const ssd_shape* shape, int path, const void* X, const void* dt,
                const float* A, const void* B, const void* C, const float* D,
                const ssd_scales* scales, void* Y, const void* initial_state, void* final_state,
                void* workspace, size_t workspace_bytes, const ssd_taps* taps, void* stream);

/* Single-token decode step: the recurrent form of the same block, one
 * position per call, continuing from a forward's final_state or an earlier
 * step's state. shape->seqlen must be 1 (or batch 0); shape->chunk is not
 * used but must be a supported value; batch * nheads <= 2^24.
 * X [B,H,P], dt [B,H], B, C [B,G,N] in shape->dtype; Y [B,H,P] in
 * shape->dtype; state [B,H,P,N] int8 (INT8, in the state scale s_S) or fp32
 * (FLOAT), read and overwritten in place with the state after the position.
 *   FLOAT: h' = exp(dt A) h + dt x B,  y = C . h' + D x  (fp32).
 *   INT8 ("Key design 2", Eq. 6 with a chunk of one position; the chunk
 *   algebra of "Overall framework" reduces to this for l = 1):
 *     Q(Decay) = min(128, RHAZ(128 exp(dt A))) decided in float64,
 *     Q(Xs) = sat127(RHAZ(fl32(fl32(dt x) inv_X))), S8 = sat127(RHAZ(fl32(
 *     fl32(Q(Xs) Q(B)) M_req))), h' = sat127(S8 + RSH7(Q(Decay) h)),
 *     y = exp(dt A) s_C s_S (Q(C) . h) + (Q(C) . Q(B)) s_C s_B dt x + D x
 *     with h the state before the position (ChunkScan1) and the single
 *     diagonal term of ChunkScan2. The state integers equal those of
 *     ssd_forward over a chunk of one position. Needs scales.
 * The state is 16-byte aligned; X, dt, B, C, Y need only element alignment
 * but are checked for 16 bytes like every other buffer. */
int ssd_decode_step(const ssd_shape* shape, int path, const void* X, const void* dt,
                    const float* A, const void* B, const void* C, const float* D,
                    const ssd_scales* scales, void* state, void* Y, void* stream);

/* SSD epilogue: the steps right after the SSD ("Overall framework": the SSD
 * output goes through RMSNorm before Out Proj; "Key design 4": the per-channel
 * mean correction, with the coefficient 0.15 of "Training strategy").
 * For every position r of Y [B, L, H*P] (shape->dtype):
 *   u = Y[r, :] + alpha * corr            (corr [H*P] fp32, may be NULL: u = Y[r, :])
 *   out[r, :] = u / sqrt(mean(u^2) + eps) * weight   (weight [H*P] fp32)
 * computed in fp32, out in shape->dtype (may alias Y). The pages apply the
 * correction at Out Proj, whose trained weights are not part of this library;
 * here it corrects the SSD output's own channels. eps >= 0 and a finite
 * alpha are required (SSD_E_SHAPE otherwise); B * L <= 2^24. */
int ssd_epilogue(const ssd_shape* shape, const void* Y, const float* corr, float alpha,
                 const float* weight, float eps, void* out, void* stream);

/* The mean correction's closed form ("Key design 4": the least-squares
 * correction of a quantised output is the per-channel mean of its error):
 * c[ch] = mean over all B * L positions of (Y_ref - Y_q)[., ch], for
 * Y_ref, Y_q [B, L, H*P] in shape->dtype (e.g. the float path's and the
 * INT8 path's outputs on calibration sequences); c [H*P] fp32. Summed in
 * float64 in a fixed order. An empty shape returns SSD_E_SHAPE. */
int ssd_mean_correction(const ssd_shape* shape, const void* Y_ref, const void* Y_q, float* c,
                        void* stream);

/* Workspace bytes ssd_forward needs (0 for an invalid shape). Host only. */
size_t ssd_workspace_bytes(const ssd_shape* shape, int path);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ssd_forward
 * with the same arguments, less workspace and workspace_bytes, whose workspace
 * is a fixed array of SSD_NOALLOC_SCRATCH_BYTES bytes of device memory that the
 * library holds on each device it runs on, from that device's first call until
 * the process ends. The call allocates nothing. It uses the current device's
 * array (the stream must belong to the current device). A problem whose
 * ssd_workspace_bytes exceeds that size returns SSD_E_TOO_LARGE and enqueues
 * nothing; with shape->schedule SSD_SCHED_AUTO the head-persistent INT8
 * schedule is taken when the chunk-parallel one would not fit. All calls on
 * one device share its array: calls that may overlap on one device (different
 * streams, or host threads without ordering) race and must not be made. The
 * results equal ssd_forward's bit for bit; nothing in the array needs to start
 * at zero. Other errors as ssd_forward. */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int ssd_forward_noalloc(const ssd_shape* shape, int path, const void* X, const void* dt,
                        const float* A, const void* B, const void* C, const float* D,
                        const ssd_scales* scales, void* Y, const void* initial_state,
                        void* final_state, const ssd_taps* taps, void* stream);

/* Calibration maxima for the static scales ("Training strategy": static
 * scales from calibration data). Over one sequence batch, raises (running
 * max) amax = [amax_B[G], amax_C[G], amax_Xs[H*P], amax_S[H*P]] (device fp32,
 * caller zero-fills before the first call) with |B|, |C| per group, |LUT * x|
 * per (h,p) and the float chunk states max(|S_k|, |H_k|) per (h,p) over
 * (b, k, n), computed on the float path in fp32. workspace: at least
 * ssd_calibrate_workspace_bytes(shape) bytes. */
int ssd_calibrate_amax(const ssd_shape* shape, const void* X, const void* dt,
                       const float* A, const void* B, const void* C, float* amax,
                       void* workspace, size_t workspace_bytes, void* stream);
size_t ssd_calibrate_workspace_bytes(const ssd_shape* shape);

/* Host-only: static scale pack from calibration maxima (host arrays).
 * amax = [amax_B[G], amax_C[G], amax_Xs[H*P], amax_S[H*P]];
 * pack (host, 4*G + 4*H*P floats) = [s_B, s_C, inv_B, inv_C (G each),
 * s_X, inv_X, s_S, M_req (H*P each)], with s = fp32(amax / 127) (1 when
 * amax is 0, an empty range), inv = fp32(1 / s), M_req = fp32(s_X s_B / s_S)
 * evaluated in float64. A maximum that is negative, NaN or infinite has no
 * scale ("Training strategy": static ranges of finite calibration
 * activations): the call then returns SSD_E_VALUE and writes nothing. */
int ssd_scales_from_amax(int64_t ngroups, int64_t nheads, int64_t headdim,
                         const float* amax, float* pack);

/* Static string for a status code. */
const char* ssd_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SSD_CHUNKED_AMD_SSD_H */
