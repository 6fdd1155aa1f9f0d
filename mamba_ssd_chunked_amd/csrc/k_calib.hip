// Calibration maxima for the static INT8 scales ("SSDi8" notes page,
// "Training strategy": static symmetric scales; axes of "Key design 3").
// Non-negative floats order like their bit patterns, so maxima are merged
// with integer atomicMax on the bits.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

__device__ __forceinline__ void atomic_max_pos(float* addr, float v) {
  atomicMax((unsigned int*)addr, __float_as_uint(v));
}

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x / kWave); ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// amax of |B| and |C| per group: grid (G, slices); rows (b, t) strided over slices.
template <int DT>
__global__ __launch_bounds__(256) void k_amax_bc(Dims d, const void* __restrict__ B,
                                                 const void* __restrict__ C,
                                                 float* __restrict__ amB,
                                                 float* __restrict__ amC) {
  __shared__ float red[4];
  const int g = blockIdx.x;
  const int64_t rows = d.B * d.L;
  float mb = 0.f, mc = 0.f;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    for (int n = threadIdx.x; n < d.N; n += blockDim.x) {
      const int64_t i = (r * d.G + g) * (int64_t)d.N + n;
      mb = fmaxf(mb, fabsf(ld_f<DT>(B, i)));
      mc = fmaxf(mc, fabsf(ld_f<DT>(C, i)));
    }
  }
  mb = block_max(mb, red);
  mc = block_max(mc, red);
  if (threadIdx.x == 0) {
    atomic_max_pos(amB + g, mb);
    atomic_max_pos(amC + g, mc);
  }
}

// amax of |lut * x| per (h, p): one block per (h, k, b), thread -> p, rows strided.
template <int DT>
__global__ __launch_bounds__(256) void k_amax_xs(Dims d, const void* __restrict__ X,
                                                 const float* __restrict__ lut,
                                                 float* __restrict__ amX) {
  __shared__ float part[256];
  const int h = blockIdx.x, k = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int P = d.P;
  const int p = threadIdx.x % P, r0 = threadIdx.x / P, rstep = 256 / P;
  float m = 0.f;
  for (int s = r0; s < d.l; s += rstep) {
    const int64_t t = (int64_t)k * d.l + s;
    if (t >= d.L) break;
    const float lv = lut[((b * d.H + h) * d.c + k) * (int64_t)d.l + s];
    m = fmaxf(m, fabsf(lv * ld_f<DT>(X, ((b * d.L + t) * d.H + h) * (int64_t)P + p)));
  }
  part[threadIdx.x] = m;
  __syncthreads();
  if (threadIdx.x < P) {
    float r = 0.f;
    for (int j = 0; j < rstep; ++j) r = fmaxf(r, part[j * P + threadIdx.x]);
    atomic_max_pos(amX + h * P + threadIdx.x, r);
  }
}

// amax of |state| per (h, p) over (b, k, n): one block per (h, k, b).
__global__ __launch_bounds__(256) void k_amax_states(Dims d, const float* __restrict__ states,
                                                     float* __restrict__ amS) {
  __shared__ float part[256];
  const int h = blockIdx.x, k = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int P = d.P, N = d.N;
  const int64_t base = ((b * d.c + k) * d.H + h) * (int64_t)P * N;
  // 256 threads: P rows, 256/P lanes per row over n
  const int p = threadIdx.x % P, j0 = threadIdx.x / P, jstep = 256 / P;
  float m = 0.f;
  for (int n = j0; n < N; n += jstep) m = fmaxf(m, fabsf(states[base + (int64_t)p * N + n]));
  part[threadIdx.x] = m;
  __syncthreads();
  if (threadIdx.x < P) {
    float r = 0.f;
    for (int j = 0; j < jstep; ++j) r = fmaxf(r, part[j * P + threadIdx.x]);
    atomic_max_pos(amS + h * P + threadIdx.x, r);
  }
}

hipError_t launch_amax_bc(const Dims& d, int dtype, const void* B, const void* C, float* amax_B,
                          float* amax_C, hipStream_t st) {
  const int64_t rows = d.B * d.L;
  const unsigned sl = (unsigned)(rows < 1024 ? rows : 1024);
  const dim3 grid(d.G, sl);
  switch (dtype) {
    case DT_F32: hipLaunchKernelGGL(k_amax_bc<DT_F32>, grid, dim3(256), 0, st, d, B, C, amax_B, amax_C); break;
    case DT_F16: hipLaunchKernelGGL(k_amax_bc<DT_F16>, grid, dim3(256), 0, st, d, B, C, amax_B, amax_C); break;
    case DT_BF16: hipLaunchKernelGGL(k_amax_bc<DT_BF16>, grid, dim3(256), 0, st, d, B, C, amax_B, amax_C); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_amax_xs(const Dims& d, int dtype, const void* X, const float* lut,
                          float* amax_X, hipStream_t st) {
  const dim3 grid(d.H, d.c, (unsigned)d.B);
  switch (dtype) {
    case DT_F32: hipLaunchKernelGGL(k_amax_xs<DT_F32>, grid, dim3(256), 0, st, d, X, lut, amax_X); break;
    case DT_F16: hipLaunchKernelGGL(k_amax_xs<DT_F16>, grid, dim3(256), 0, st, d, X, lut, amax_X); break;
    case DT_BF16: hipLaunchKernelGGL(k_amax_xs<DT_BF16>, grid, dim3(256), 0, st, d, X, lut, amax_X); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_amax_states(const Dims& d, const float* states, float* amax_S, hipStream_t st) {
  const dim3 grid(d.H, d.c, (unsigned)d.B);
  hipLaunchKernelGGL(k_amax_states, grid, dim3(256), 0, st, d, states, amax_S);
  return hipGetLastError();
}

}  // namespace ssd
