// C ABI of the SSD chunked forward: argument validation (host only, before
// any launch), workspace carving and dispatch to the HIP kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/ssd.h"
#include "ssd_launch.hpp"

using ssd::Dims;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Validates the shape; fills d. *empty is set for batch == 0 or seqlen == 0.
int check_shape(const ssd_shape* s, Dims* d, bool* empty) {
  if (!s) return SSD_E_NULL;
  if (s->schedule < SSD_SCHED_AUTO || s->schedule > SSD_SCHED_CHUNK) return SSD_E_SHAPE;
  if (s->batch < 0 || s->seqlen < 0) return SSD_E_SHAPE;
  if (s->nheads <= 0 || s->headdim <= 0 || s->dstate <= 0 || s->ngroups <= 0 || s->chunk <= 0)
    return SSD_E_SHAPE;
  if (s->nheads % s->ngroups != 0) return SSD_E_SHAPE;
  if (s->dtype < SSD_DTYPE_F32 || s->dtype > SSD_DTYPE_BF16) return SSD_E_UNSUPPORTED;
  if (s->chunk != 64 && s->chunk != 128 && s->chunk != 256) return SSD_E_UNSUPPORTED;
  if (s->headdim != 16 && s->headdim != 32 && s->headdim != 64) return SSD_E_UNSUPPORTED;
  if (s->dstate != 16 && s->dstate != 32 && s->dstate != 64 && s->dstate != 128)
    return SSD_E_UNSUPPORTED;
  // grid limits: H in x, chunks in y, batch in z
  const int64_t c = s->seqlen / s->chunk + (s->seqlen % s->chunk != 0);  // no overflow near INT64_MAX
  if (s->nheads > 65535 || s->batch > 65535 || c > 65535) return SSD_E_SHAPE;
  // every element count must fit an int64 byte offset
  int64_t t;
  if (!mul_ok(s->batch, s->seqlen, &t) || !mul_ok(t, s->nheads, &t) ||
      !mul_ok(t, s->headdim, &t) || !mul_ok(t, 16, &t))
    return SSD_E_SHAPE;
  int64_t u;
  if (!mul_ok(s->batch, c, &u) || !mul_ok(u, s->nheads, &u) || !mul_ok(u, s->headdim, &u) ||
      !mul_ok(u, s->dstate, &u) || !mul_ok(u, 16, &u))
    return SSD_E_SHAPE;
  int64_t v;
  if (!mul_ok(s->batch, c, &v) || !mul_ok(v, s->ngroups, &v) || !mul_ok(v, s->chunk, &v) ||
      !mul_ok(v, s->chunk, &v) || !mul_ok(v, 16, &v))
    return SSD_E_SHAPE;
  d->B = s->batch;
  d->L = s->seqlen;
  d->H = (int)s->nheads;
  d->P = (int)s->headdim;
  d->N = (int)s->dstate;
  d->G = (int)s->ngroups;
  d->l = (int)s->chunk;
  d->c = (int)c;
  d->hpg = d->H / d->G;
  d->sched = s->schedule;
  *empty = (s->batch == 0 || s->seqlen == 0);
  return SSD_OK;
}

// The module calls and the decode step compute the float and INT8 paths.
int check_path(int path) {
  return (path == SSD_PATH_FLOAT || path == SSD_PATH_INT8) ? SSD_OK : SSD_E_UNSUPPORTED;
}

// ssd_forward also runs the two Table 5 ablation rows.
int check_forward_path(int path) {
  return (path >= SSD_PATH_FLOAT && path <= SSD_PATH_ABL_RECON) ? SSD_OK : SSD_E_UNSUPPORTED;
}

// Each required pointer must be non-NULL and 16-byte aligned.
int check_ptrs(std::initializer_list<const void*> req) {
  for (const void* p : req)
    if (!p) return SSD_E_NULL;
  for (const void* p : req)
    if (!aligned16(p)) return SSD_E_ALIGN;
  return SSD_OK;
}

int check_opt(std::initializer_list<const void*> opt) {
  for (const void* p : opt)
    if (p && !aligned16(p)) return SSD_E_ALIGN;
  return SSD_OK;
}

// Scale arrays are read element-wise: non-NULL and 4-byte aligned. Which
// arrays a path reads: INT8 the first seven; the "Q(X) only" row s_Xq and
// inv_Xq; the "reconstruction + B,C" row the first seven and s_X.
int check_scales(const ssd_scales* sc, int path = SSD_PATH_INT8) {
  if (!sc) return SSD_E_NULL;
  const void* req[8];
  int n = 0;
  if (path == SSD_PATH_ABL_QX) {
    req[n++] = sc->s_Xq;
    req[n++] = sc->inv_Xq;
  } else {
    const void* base[] = {sc->s_B, sc->s_C, sc->inv_B, sc->inv_C, sc->inv_X, sc->s_S, sc->M_req};
    for (const void* p : base) req[n++] = p;
    if (path == SSD_PATH_ABL_RECON) req[n++] = sc->s_X;
  }
  for (int i = 0; i < n; ++i)
    if (!req[i]) return SSD_E_NULL;
  for (int i = 0; i < n; ++i)
    if (reinterpret_cast<uintptr_t>(req[i]) & 3u) return SSD_E_ALIGN;
  return SSD_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_E_HIP; }

ssd::ScalePtrs scale_ptrs(const ssd_scales* sc) {
  ssd::ScalePtrs p{};
  if (sc) {
    p.s_B = sc->s_B;
    p.s_C = sc->s_C;
    p.inv_B = sc->inv_B;
    p.inv_C = sc->inv_C;
    p.inv_X = sc->inv_X;
    p.s_S = sc->s_S;
    p.M_req = sc->M_req;
    p.s_X = sc->s_X;
    p.s_Xq = sc->s_Xq;
    p.inv_Xq = sc->inv_Xq;
  }
  return p;
}

// Byte sizes of the intermediates.
struct Sizes {
  size_t qbc, cs, qd, st_i8, st_f32, cb;
};
Sizes sizes_of(const Dims& d) {
  Sizes z;
  z.qbc = (size_t)d.B * d.L * d.G * d.N;
  z.cs = (size_t)d.B * d.H * d.c * d.l * sizeof(float);
  z.qd = (size_t)d.B * d.H * d.c;
  z.st_i8 = (size_t)d.B * d.c * d.H * d.P * d.N;
  z.st_f32 = z.st_i8 * sizeof(float);
  z.cb = (size_t)d.B * d.c * d.G * d.l * d.l * sizeof(int32_t);
  return z;
}

// Workspace of the module-by-module composition of ssd_forward.
size_t modular_ws_bytes(const Dims& d, int path) {
  const Sizes z = sizes_of(d);
  size_t n = 2 * align_up(z.cs) + align_up(z.cb);
  switch (path) {
    case SSD_PATH_INT8: n += 2 * align_up(z.qbc) + align_up(z.qd) + align_up(z.st_i8); break;
    case SSD_PATH_ABL_QX: n += align_up((size_t)d.B * d.L * d.H * d.P) + align_up(z.st_f32); break;
    case SSD_PATH_ABL_RECON: n += 2 * align_up(z.qbc) + align_up(z.st_f32); break;
    default: n += align_up(z.st_f32); break;
  }
  return n;
}

// The two Table 5 ablation rows ("SSDi8" notes page, experiments, Table 5),
// composed from the module kernels:
//   "Q(X) only"                 Q(X) once per (h,p); float modules on Q(X) s_Xq;
//   "reconstruction + B,C"      Q(B), Q(C); ChunkState on INT8 (S32), dequantised
//                               to fp32 with s_X s_B; float StatePassing; float
//                               ChunkBMM on B, C; ChunkScan with an INT8 Scan1
//                               (passed states quantised with s_S) and a float Scan2.
int forward_ablation(const Dims& d, int dtype, int path, const void* X, const void* dt,
                     const float* A, const void* B, const void* C, const float* D,
                     const ssd::ScalePtrs& sp, void* Y, void* final_state, void* workspace,
                     hipStream_t st) {
  const Sizes z = sizes_of(d);
  char* w = (char*)workspace;
  float* dAcs = (float*)w;
  w += align_up(z.cs);
  float* lut = (float*)w;
  w += align_up(z.cs);
  float* CB = (float*)w;
  w += align_up(z.cb);
  if (path == SSD_PATH_ABL_QX) {
    int8_t* qx = (int8_t*)w;
    w += align_up((size_t)d.B * d.L * d.H * d.P);
    float* states = (float*)w;
    if (ssd::launch_quantize_x(d, dtype, X, sp.inv_Xq, qx, st)) return SSD_E_HIP;
    if (ssd::launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, nullptr, st)) return SSD_E_HIP;
    if (ssd::launch_chunk_state(d, dtype, ssd::kModeQx, qx, lut, B, nullptr, nullptr, sp.s_Xq, nullptr,
                                states, nullptr, nullptr, st))
      return SSD_E_HIP;
    if (ssd::launch_state_passing(d, false, states, dAcs, nullptr, nullptr, final_state, st)) return SSD_E_HIP;
    if (ssd::launch_chunk_bmm(d, dtype, false, C, B, CB, st)) return SSD_E_HIP;
    if (ssd::launch_chunk_scan(d, dtype, ssd::kModeQx, qx, dt, dAcs, C, CB, states, nullptr, D, nullptr,
                               nullptr, nullptr, sp.s_Xq, Y, st))
      return SSD_E_HIP;
    return SSD_OK;
  }
  int8_t* qB = (int8_t*)w;
  w += align_up(z.qbc);
  int8_t* qC = (int8_t*)w;
  w += align_up(z.qbc);
  float* states = (float*)w;
  if (ssd::launch_quantize_bc(d, dtype, B, C, sp.inv_B, sp.inv_C, qB, qC, st)) return SSD_E_HIP;
  if (ssd::launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, nullptr, st)) return SSD_E_HIP;
  if (ssd::launch_chunk_state(d, dtype, ssd::kModeRecon, X, lut, qB, sp.inv_X, nullptr, sp.s_X, sp.s_B,
                              states, nullptr, nullptr, st))
    return SSD_E_HIP;
  if (ssd::launch_state_passing(d, false, states, dAcs, nullptr, nullptr, final_state, st)) return SSD_E_HIP;
  if (ssd::launch_chunk_bmm(d, dtype, false, C, B, CB, st)) return SSD_E_HIP;
  if (ssd::launch_chunk_scan(d, dtype, ssd::kModeRecon, X, dt, dAcs, qC, CB, states, nullptr, D, sp.s_C,
                             sp.s_B, sp.s_S, nullptr, Y, st))
    return SSD_E_HIP;
  return SSD_OK;
}

// seqlen == 0 with batch > 0: the state after no positions is the initial state
// (zero without one), so final_state, when given, receives it.
int zero_length_state(const Dims& d, size_t elem, const void* initial_state, void* final_state,
                      hipStream_t st) {
  if (d.B == 0 || d.L != 0 || !final_state) return SSD_OK;
  const size_t bytes = (size_t)d.B * d.H * d.P * d.N * elem;
  if (initial_state)
    return hip_status(hipMemcpyAsync(final_state, initial_state, bytes, hipMemcpyDeviceToDevice, st));
  return hip_status(ssd::launch_zero_fill(final_state, bytes, st));
}

}  // namespace

extern "C" {

const char* ssd_status_string(int status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_E_NULL: return "a required pointer is NULL";
    case SSD_E_SHAPE: return "invalid shape (sizes, H % G, or size overflow)";
    case SSD_E_UNSUPPORTED: return "unsupported chunk, headdim, dstate, dtype or path";
    case SSD_E_ALIGN: return "a buffer is not 16-byte aligned";
    case SSD_E_WORKSPACE: return "workspace too small";
    case SSD_E_HIP: return "HIP runtime error";
    case SSD_E_INTERNAL: return "internal error";
    case SSD_E_VALUE: return "a calibration maximum is negative, NaN or infinite";
    case SSD_E_TOO_LARGE: return "problem needs more workspace than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int ssd_quantize_bc(const ssd_shape* shape, const void* B, const void* C,
                    const ssd_scales* scales, int8_t* qB, int8_t* qC, void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_scales(scales))) return rc;
  if ((rc = check_ptrs({B, C, qB, qC}))) return rc;
  if (empty) return SSD_OK;
  return hip_status(ssd::launch_quantize_bc(d, shape->dtype, B, C, scales->inv_B, scales->inv_C,
                                            qB, qC, (hipStream_t)stream));
}

int ssd_chunk_cumsum(const ssd_shape* shape, const void* dt, const float* A, float* dAcs,
                     float* lut, uint8_t* qdecay, void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_ptrs({dt, A, dAcs}))) return rc;
  if ((rc = check_opt({lut, qdecay}))) return rc;
  if (empty) return SSD_OK;
  return hip_status(ssd::launch_chunk_cumsum(d, shape->dtype, dt, A, dAcs, lut, qdecay,
                                             (hipStream_t)stream));
}

int ssd_chunk_state(const ssd_shape* shape, int path, const void* X, const float* lut,
                    const void* Bq, const ssd_scales* scales, void* states,
                    const ssd_taps* taps, void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_path(path))) return rc;
  const bool i8 = path == SSD_PATH_INT8;
  if ((rc = check_ptrs({X, lut, Bq, states}))) return rc;
  if (i8 && (rc = check_scales(scales))) return rc;
  int8_t* tq = (i8 && taps) ? taps->q_xs : nullptr;
  int32_t* ts = (i8 && taps) ? taps->s32 : nullptr;
  if ((rc = check_opt({tq, ts}))) return rc;
  if (empty) return SSD_OK;
  return hip_status(ssd::launch_chunk_state(d, shape->dtype, i8 ? ssd::kModeInt8 : ssd::kModeFloat,
                                            X, lut, Bq, i8 ? scales->inv_X : nullptr,
                                            i8 ? scales->M_req : nullptr, nullptr, nullptr, states,
                                            tq, ts, (hipStream_t)stream));
}

int ssd_state_passing(const ssd_shape* shape, int path, void* states, const float* dAcs,
                      const uint8_t* qdecay, const void* initial_state, void* final_state,
                      void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_path(path))) return rc;
  const bool i8 = path == SSD_PATH_INT8;
  if ((rc = check_ptrs({states, i8 ? (const void*)qdecay : (const void*)dAcs}))) return rc;
  if ((rc = check_opt({initial_state, final_state}))) return rc;
  if (empty) return zero_length_state(d, i8 ? 1 : 4, initial_state, final_state, (hipStream_t)stream);
  return hip_status(ssd::launch_state_passing(d, i8, states, dAcs, qdecay, initial_state,
                                              final_state, (hipStream_t)stream));
}

int ssd_chunk_bmm(const ssd_shape* shape, int path, const void* Cq, const void* Bq, void* CB,
                  void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_path(path))) return rc;
  if ((rc = check_ptrs({Cq, Bq, CB}))) return rc;
  if (empty) return SSD_OK;
  return hip_status(ssd::launch_chunk_bmm(d, shape->dtype, path == SSD_PATH_INT8, Cq, Bq, CB,
                                          (hipStream_t)stream));
}

int ssd_chunk_scan(const ssd_shape* shape, int path, const void* X, const void* dt,
                   const float* dAcs, const void* Cq, const void* CB, const void* states,
                   const void* initial_state, const float* D, const ssd_scales* scales, void* Y,
                   void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_path(path))) return rc;
  const bool i8 = path == SSD_PATH_INT8;
  if ((rc = check_ptrs({X, dt, dAcs, Cq, CB, states, D, Y}))) return rc;
  if ((rc = check_opt({initial_state}))) return rc;
  if (i8 && (rc = check_scales(scales))) return rc;
  if (empty) return SSD_OK;
  return hip_status(ssd::launch_chunk_scan(d, shape->dtype, i8 ? ssd::kModeInt8 : ssd::kModeFloat,
                                           X, dt, dAcs, Cq, CB, states, initial_state, D,
                                           i8 ? scales->s_C : nullptr,
                                           i8 ? scales->s_B : nullptr,
                                           i8 ? scales->s_S : nullptr, nullptr, Y,
                                           (hipStream_t)stream));
}

size_t ssd_workspace_bytes(const ssd_shape* shape, int path) {
  Dims d;
  bool empty;
  if (check_shape(shape, &d, &empty) != SSD_OK || check_forward_path(path) != SSD_OK) return 0;
  const bool i8 = path == SSD_PATH_INT8;
  if (empty) return 0;
  if (path <= SSD_PATH_INT8 && ssd::fused_supported(d, shape->dtype, i8))
    return ssd::fused_workspace_bytes(d, i8);
  return modular_ws_bytes(d, path);
}

int ssd_forward(const ssd_shape* shape, int path, const void* X, const void* dt, const float* A,
                const void* B, const void* C, const float* D, const ssd_scales* scales, void* Y,
                const void* initial_state, void* final_state, void* workspace,
                size_t workspace_bytes, const ssd_taps* taps, void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_forward_path(path))) return rc;
  const bool i8 = path == SSD_PATH_INT8;
  const bool abl = path == SSD_PATH_ABL_QX || path == SSD_PATH_ABL_RECON;
  if ((rc = check_ptrs({X, dt, A, B, C, D, Y}))) return rc;
  if (path != SSD_PATH_FLOAT && (rc = check_scales(scales, path))) return rc;
  if (abl && initial_state) return SSD_E_UNSUPPORTED;
  int8_t* tq = (i8 && taps) ? taps->q_xs : nullptr;
  int32_t* ts = (i8 && taps) ? taps->s32 : nullptr;
  int8_t* t8 = (i8 && taps) ? taps->s8_local : nullptr;
  int8_t* tp = (i8 && taps) ? taps->passed : nullptr;
  if ((rc = check_opt({initial_state, final_state, workspace, tq, ts, t8, tp}))) return rc;
  if (empty) return zero_length_state(d, i8 ? 1 : 4, initial_state, final_state, (hipStream_t)stream);
  const size_t need = ssd_workspace_bytes(shape, path);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SSD_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int dtype = shape->dtype;
  const ssd::ScalePtrs sp = scale_ptrs(scales);

  if (abl) return forward_ablation(d, dtype, path, X, dt, A, B, C, D, sp, Y, final_state, workspace, st);

  if (ssd::fused_supported(d, dtype, i8)) {
    hipError_t e = ssd::launch_forward_fused(d, dtype, i8, X, dt, A, B, C, D, sp, Y, initial_state,
                                             final_state, workspace, tq, ts, t8, tp, st);
    return hip_status(e);
  }

  // module-by-module composition
  const Sizes z = sizes_of(d);
  char* w = (char*)workspace;
  float* dAcs = (float*)w;
  w += align_up(z.cs);
  float* lut = (float*)w;
  w += align_up(z.cs);
  void* CB = w;
  w += align_up(z.cb);
  hipError_t e;
  if (i8) {
    int8_t* qB = (int8_t*)w;
    w += align_up(z.qbc);
    int8_t* qC = (int8_t*)w;
    w += align_up(z.qbc);
    uint8_t* qd = (uint8_t*)w;
    w += align_up(z.qd);
    int8_t* states = (int8_t*)w;
    if ((e = ssd::launch_quantize_bc(d, dtype, B, C, sp.inv_B, sp.inv_C, qB, qC, st))) return SSD_E_HIP;
    if ((e = ssd::launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, qd, st))) return SSD_E_HIP;
    if ((e = ssd::launch_chunk_state(d, dtype, ssd::kModeInt8, X, lut, qB, sp.inv_X, sp.M_req, nullptr,
                                     nullptr, states, tq, ts, st)))
      return SSD_E_HIP;
    if (t8 && (e = hipMemcpyAsync(t8, states, z.st_i8, hipMemcpyDeviceToDevice, st))) return SSD_E_HIP;
    if ((e = ssd::launch_state_passing(d, true, states, dAcs, qd, initial_state, final_state, st)))
      return SSD_E_HIP;
    if (tp && (e = hipMemcpyAsync(tp, states, z.st_i8, hipMemcpyDeviceToDevice, st))) return SSD_E_HIP;
    if ((e = ssd::launch_chunk_bmm(d, dtype, true, qC, qB, CB, st))) return SSD_E_HIP;
    if ((e = ssd::launch_chunk_scan(d, dtype, ssd::kModeInt8, X, dt, dAcs, qC, CB, states, initial_state,
                                    D, sp.s_C, sp.s_B, sp.s_S, nullptr, Y, st)))
      return SSD_E_HIP;
  } else {
    float* states = (float*)w;
    if ((e = ssd::launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, nullptr, st))) return SSD_E_HIP;
    if ((e = ssd::launch_chunk_state(d, dtype, ssd::kModeFloat, X, lut, B, nullptr, nullptr, nullptr,
                                     nullptr, states, nullptr, nullptr, st)))
      return SSD_E_HIP;
    if ((e = ssd::launch_state_passing(d, false, states, dAcs, nullptr, initial_state, final_state, st)))
      return SSD_E_HIP;
    if ((e = ssd::launch_chunk_bmm(d, dtype, false, C, B, CB, st))) return SSD_E_HIP;
    if ((e = ssd::launch_chunk_scan(d, dtype, ssd::kModeFloat, X, dt, dAcs, C, CB, states, initial_state,
                                    D, nullptr, nullptr, nullptr, nullptr, Y, st)))
      return SSD_E_HIP;
  }
  return SSD_OK;
}

int ssd_decode_step(const ssd_shape* shape, int path, const void* X, const void* dt,
                    const float* A, const void* B, const void* C, const float* D,
                    const ssd_scales* scales, void* state, void* Y, void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_path(path))) return rc;
  if (d.B > 0 && d.L != 1) return SSD_E_SHAPE;
  // one wave per (batch, head): keep the grid's thread count below 2^32
  if (d.B * (int64_t)d.H > (int64_t)1 << 24) return SSD_E_SHAPE;
  const bool i8 = path == SSD_PATH_INT8;
  if ((rc = check_ptrs({X, dt, A, B, C, D, state, Y}))) return rc;
  if (i8 && (rc = check_scales(scales))) return rc;
  if (empty) return SSD_OK;
  return hip_status(ssd::launch_decode_step(d, shape->dtype, i8, X, dt, A, B, C, D,
                                            scale_ptrs(scales), state, Y, (hipStream_t)stream));
}

int ssd_epilogue(const ssd_shape* shape, const void* Y, const float* corr, float alpha,
                 const float* weight, float eps, void* out, void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_ptrs({Y, weight, out}))) return rc;
  if ((rc = check_opt({corr}))) return rc;
  if (!(eps >= 0.0f) || !std::isfinite(alpha)) return SSD_E_SHAPE;
  // a workgroup per four positions: keeps the grid far below 2^32 threads
  if (d.B * d.L > (int64_t)1 << 24) return SSD_E_SHAPE;
  if (empty) return SSD_OK;
  return hip_status(ssd::launch_epilogue(d, shape->dtype, Y, corr, alpha, weight, eps, out,
                                         (hipStream_t)stream));
}

int ssd_mean_correction(const ssd_shape* shape, const void* Y_ref, const void* Y_q, float* c,
                        void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_ptrs({Y_ref, Y_q, c}))) return rc;
  if (empty) return SSD_E_SHAPE;  // the mean of no positions is undefined
  return hip_status(ssd::launch_mean_correction(d, shape->dtype, Y_ref, Y_q, c, (hipStream_t)stream));
}

size_t ssd_calibrate_workspace_bytes(const ssd_shape* shape) {
  Dims d;
  bool empty;
  if (check_shape(shape, &d, &empty) != SSD_OK || empty) return 0;
  const Sizes z = sizes_of(d);
  return 2 * align_up(z.cs) + align_up(z.st_f32);
}

int ssd_calibrate_amax(const ssd_shape* shape, const void* X, const void* dt, const float* A,
                       const void* B, const void* C, float* amax, void* workspace,
                       size_t workspace_bytes, void* stream) {
  Dims d;
  bool empty;
  int rc = check_shape(shape, &d, &empty);
  if (rc) return rc;
  if ((rc = check_ptrs({X, dt, A, B, C, amax}))) return rc;
  if ((rc = check_opt({workspace}))) return rc;
  if (empty) return SSD_OK;
  const size_t need = ssd_calibrate_workspace_bytes(shape);
  if (!workspace || workspace_bytes < need) return SSD_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const Sizes z = sizes_of(d);
  char* w = (char*)workspace;
  float* dAcs = (float*)w;
  w += align_up(z.cs);
  float* lut = (float*)w;
  w += align_up(z.cs);
  float* states = (float*)w;
  float* amB = amax;
  float* amC = amax + d.G;
  float* amX = amax + 2 * d.G;
  float* amS = amX + (size_t)d.H * d.P;
  const int dtype = shape->dtype;
  if (ssd::launch_amax_bc(d, dtype, B, C, amB, amC, st)) return SSD_E_HIP;
  if (ssd::launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, nullptr, st)) return SSD_E_HIP;
  if (ssd::launch_amax_xs(d, dtype, X, lut, amX, st)) return SSD_E_HIP;
  if (ssd::launch_chunk_state(d, dtype, ssd::kModeFloat, X, lut, B, nullptr, nullptr, nullptr, nullptr,
                              states, nullptr, nullptr, st))
    return SSD_E_HIP;
  if (ssd::launch_amax_states(d, states, amS, st)) return SSD_E_HIP;
  if (ssd::launch_state_passing(d, false, states, dAcs, nullptr, nullptr, nullptr, st)) return SSD_E_HIP;
  if (ssd::launch_amax_states(d, states, amS, st)) return SSD_E_HIP;
  return SSD_OK;
}

int ssd_scales_from_amax(int64_t ngroups, int64_t nheads, int64_t headdim, const float* amax,
                         float* pack) {
  if (!amax || !pack) return SSD_E_NULL;
  if (ngroups <= 0 || nheads <= 0 || headdim <= 0 || nheads % ngroups) return SSD_E_SHAPE;
  const int64_t G = ngroups, HP = nheads * headdim, hpg = nheads / ngroups;
  // every maximum is checked before anything is written
  for (int64_t i = 0; i < 2 * G + 2 * HP; ++i)
    if (!std::isfinite(amax[i]) || amax[i] < 0.f) return SSD_E_VALUE;
  auto step = [](float a) -> float {
    const double v = (double)a;
    if (!(v > 0.0)) return 1.0f;  // an empty range
    return (float)(v / 127.0);
  };
  float* s_B = pack;
  float* s_C = pack + G;
  float* inv_B = pack + 2 * G;
  float* inv_C = pack + 3 * G;
  float* s_X = pack + 4 * G;
  float* inv_X = s_X + HP;
  float* s_S = inv_X + HP;
  float* M_req = s_S + HP;
  for (int64_t g = 0; g < G; ++g) {
    s_B[g] = step(amax[g]);
    s_C[g] = step(amax[G + g]);
    inv_B[g] = (float)(1.0 / (double)s_B[g]);
    inv_C[g] = (float)(1.0 / (double)s_C[g]);
  }
  for (int64_t i = 0; i < HP; ++i) {
    s_X[i] = step(amax[2 * G + i]);
    s_S[i] = step(amax[2 * G + HP + i]);
    inv_X[i] = (float)(1.0 / (double)s_X[i]);
    const int64_t g = (i / headdim) / hpg;
    M_req[i] = (float)((double)s_X[i] * (double)s_B[g] / (double)s_S[i]);
  }
  return SSD_OK;
}

}  // extern "C"
