// Internal launch interface between the C ABI (ssd_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Validated problem dimensions. c = ceil(L / l); hpg = H / G.
struct Dims {
  int64_t B, L;
  int H, P, N, G, l, c, hpg;
  int sched;  // kSched* of the shape (INT8 forward only)
};

struct ScalePtrs {
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
};

// INT8 forward schedules; the values equal the C ABI's SSD_SCHED_* codes.
enum { kSchedAuto = 0, kSchedHead = 1, kSchedChunk = 2 };

// Module-kernel modes; the values equal the C ABI's SSD_PATH_* codes.
enum { kModeFloat = 0, kModeInt8 = 1, kModeQx = 2, kModeRecon = 3 };

hipError_t launch_quantize_bc(const Dims& d, int dtype, const void* B, const void* C,
                              const float* inv_B, const float* inv_C, int8_t* qB, int8_t* qC,
                              hipStream_t st);
hipError_t launch_chunk_cumsum(const Dims& d, int dtype, const void* dt, const float* A,
                               float* dAcs, float* lut, uint8_t* qdecay, hipStream_t st);
hipError_t launch_quantize_x(const Dims& d, int dtype, const void* X, const float* inv_Xq,
                             int8_t* qx, hipStream_t st);
hipError_t launch_chunk_state(const Dims& d, int dtype, int mode, const void* X,
                              const float* lut, const void* Bq, const float* inv_X,
                              const float* M_req, const float* sx, const float* sb, void* states,
                              int8_t* tap_qxs, int32_t* tap_s32, hipStream_t st);
hipError_t launch_state_passing(const Dims& d, bool int8, void* states, const float* dAcs,
                                const uint8_t* qdecay, const void* init, void* final_state,
                                hipStream_t st);
hipError_t launch_chunk_bmm(const Dims& d, int dtype, bool int8, const void* Cq,
                            const void* Bq, void* CB, hipStream_t st);
hipError_t launch_chunk_scan(const Dims& d, int dtype, int mode, const void* X, const void* dt,
                             const float* dAcs, const void* Cq, const void* CB,
                             const void* states, const void* init, const float* D,
                             const float* s_C, const float* s_B, const float* s_S, const float* sx,
                             void* Y, hipStream_t st);

// Fused forward (defined in k_fused.hip). Returns hipErrorNotSupported when the
// fused kernels do not cover the shape; the caller then composes the modules.
hipError_t launch_forward_fused(const Dims& d, int dtype, bool int8, const void* X,
                                const void* dt, const float* A, const void* B, const void* C,
                                const float* D, const ScalePtrs& sc, void* Y,
                                const void* initial_state, void* final_state, void* ws,
                                int8_t* tap_qxs, int32_t* tap_s32, int8_t* tap_s8,
                                int8_t* tap_passed, hipStream_t st);
size_t fused_workspace_bytes(const Dims& d, bool int8);
bool fused_supported(const Dims& d, int dtype, bool int8);

// Fused INT8 forward (k_fused_i8.hip): ChunkCumsum, the per-(batch, chunk,
// group) B/C quantisation and ChunkBMM, then the per-head main kernel.
hipError_t launch_forward_i8(const Dims& d, int dtype, const void* X, const void* dt, const float* A,
                             const void* B, const void* C, const float* D, const ScalePtrs& sc, void* Y,
                             const void* init, void* final_state, void* ws, int8_t* tap_qxs, int32_t* tap_s32,
                             int8_t* tap_s8, int8_t* tap_passed, hipStream_t st);
size_t fused_i8_workspace_bytes(const Dims& d);
size_t i8_states_offset(const Dims& d);
bool use_chunked_i8(const Dims& d);

// Chunk-parallel schedule of the fused INT8 forward (k_chunked_i8.hip), run on
// the preparation launch's outputs; states: int8 [B, c, H, P, N] workspace.
hipError_t launch_chunked_i8(const Dims& d, int dtype, const void* X, const void* dt, const int8_t* qC,
                             const int8_t* qbt, const uint16_t* cbf, const float* dAcs, const float* lut,
                             const uint8_t* qdecay, const float* D, const ScalePtrs& sc, void* Y, const void* init,
                             void* final_state, int8_t* states, int8_t* tap_qxs, int32_t* tap_s32, int8_t* tap_s8,
                             int8_t* tap_passed, hipStream_t st);
size_t chunked_i8_states_bytes(const Dims& d);

// Calibration helpers (k_calib.hip).
hipError_t launch_amax_bc(const Dims& d, int dtype, const void* B, const void* C, float* amax_B,
                          float* amax_C, hipStream_t st);
hipError_t launch_amax_xs(const Dims& d, int dtype, const void* X, const float* lut,
                          float* amax_X, hipStream_t st);
hipError_t launch_amax_states(const Dims& d, const float* states, float* amax_S, hipStream_t st);

// Compute units of the current device (0 if unknown).
int cu_count();

// Single-token decode step (seqlen 1), state [B,H,P,N] updated in place.
hipError_t launch_decode_step(const Dims& d, int dtype, bool int8, const void* X, const void* dt,
                              const float* A, const void* B, const void* C, const float* D,
                              const ScalePtrs& sc, void* state, void* Y, hipStream_t st);

// SSD epilogue: RMSNorm with the optional mean correction (k_epilogue.hip).
hipError_t launch_epilogue(const Dims& d, int dtype, const void* Y, const float* corr, float alpha,
                           const float* weight, float eps, void* out, hipStream_t st);
hipError_t launch_mean_correction(const Dims& d, int dtype, const void* Yr, const void* Yq, float* c,
                                  hipStream_t st);

// Zero fill of a device buffer by a kernel (so that a captured graph holds no
// memset node); bytes is a multiple of 16 and p 16-byte aligned.
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st);

}  // namespace ssd
