// The steps right after the SSD ("SSDi8" notes page, "Overall framework": the
// SSD output goes through RMSNorm before Out Proj; "Key design 4": the
// per-channel mean correction, applied with coefficient 0.15 as the "Training
// strategy" section fixes):
//
//   ssd_epilogue         out[r, :] = RMSNorm(Y[r, :] + alpha c) * weight over the
//                        H*P channels of each position r;
//   ssd_mean_correction  c[ch] = mean over the positions of (Y_ref - Y_q)[., ch],
//                        the closed-form least-squares correction.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {
namespace {

constexpr int kEpThreads = 256;
constexpr int kEpVec = 8;  // elements per vector access

// One workgroup per kEpRows positions. The weight and alpha * corr vectors a
// thread needs are loaded once per workgroup and kept in registers for all its
// rows (they were the larger part of the cache traffic when every position
// re-read them). Each thread keeps up to kMaxV vectors of every row in
// registers between the sum of squares and the normalised write: rows of up
// to 256 * kMaxV * 8 = 6144 channels are read once; longer rows re-read the
// rest, which the cache serves. The rows are read and written once, so those
// loads and stores carry the non-temporal hint. out may be Y itself: each
// element is read before the same thread overwrites it, after the whole row
// has been summed.
constexpr int kEpRows = 2;
constexpr int kMaxV = 3;

template <int DT>
__device__ __forceinline__ void ld8_nt(const void* p, int64_t i, float out[8]) {
  if constexpr (DT == DT_F32) {
    typedef float v4f_ __attribute__((ext_vector_type(4)));
    const v4f_ a = __builtin_nontemporal_load((const v4f_*)((const float*)p + i));
    const v4f_ b = __builtin_nontemporal_load((const v4f_*)((const float*)p + i) + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[j] = a[j];
      out[4 + j] = b[j];
    }
  } else {
    typedef uint32_t v4u_ __attribute__((ext_vector_type(4)));
    const v4u_ v = __builtin_nontemporal_load((const v4u_*)((const u16*)p + i));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = Store<DT>::to_f(__builtin_bit_cast(typename Store<DT>::T, (u16)(v[j] & 0xffff)));
      out[2 * j + 1] = Store<DT>::to_f(__builtin_bit_cast(typename Store<DT>::T, (u16)(v[j] >> 16)));
    }
  }
}

template <int DT>
__device__ __forceinline__ void st8_nt(void* p, int64_t i, const float o[8]) {
  if constexpr (DT == DT_F32) {
    typedef float v4f_ __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store((v4f_){o[0], o[1], o[2], o[3]}, (v4f_*)((float*)p + i));
    __builtin_nontemporal_store((v4f_){o[4], o[5], o[6], o[7]}, (v4f_*)((float*)p + i) + 1);
  } else {
    typedef uint32_t v4u_ __attribute__((ext_vector_type(4)));
    v4u_ w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = pack2<DT>(o[2 * j], o[2 * j + 1]);
    __builtin_nontemporal_store(w, (v4u_*)((u16*)p + i));
  }
}

template <int DT>
__global__ __launch_bounds__(kEpThreads) void k_epilogue(const void* Y,
                                                         const float* __restrict__ corr,
                                                         float alpha,
                                                         const float* __restrict__ weight,
                                                         float eps, void* out,
                                                         int Dc, int64_t rows) {
  __shared__ float red[kEpRows][kEpThreads / kWave];
  const int64_t row0 = (int64_t)blockIdx.x * kEpRows;
  const int nr = (int)min((int64_t)kEpRows, rows - row0);  // rows of this workgroup (uniform)
  const int nv = Dc / kEpVec;
  // without a correction the weight array stands in for it with a zero
  // coefficient, so every access is an unconditional vector load
  const float* const cp = corr ? corr : weight;
  const float al = corr ? alpha : 0.f;
  float wv[kMaxV][kEpVec], cv[kMaxV][kEpVec];
#pragma unroll
  for (int i = 0; i < kMaxV; ++i) {
    const int v = threadIdx.x + i * kEpThreads;
    if (v < nv) {
      ld8_f<DT_F32>(weight, (int64_t)v * kEpVec, wv[i]);
      ld8_f<DT_F32>(cp, (int64_t)v * kEpVec, cv[i]);
    }
  }
  float u[kEpRows][kMaxV][kEpVec];
  float ss[kEpRows];
#pragma unroll
  for (int r = 0; r < kEpRows; ++r) {
    ss[r] = 0.f;
    if (r < nr) {
#pragma unroll
      for (int i = 0; i < kMaxV; ++i) {
        const int v = threadIdx.x + i * kEpThreads;
        if (v < nv) ld8_nt<DT>(Y, (row0 + r) * (int64_t)Dc + (int64_t)v * kEpVec, u[r][i]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kEpRows; ++r) {
    if (r < nr) {
#pragma unroll
      for (int i = 0; i < kMaxV; ++i) {
        const int v = threadIdx.x + i * kEpThreads;
        if (v < nv) {
#pragma unroll
          for (int j = 0; j < kEpVec; ++j) {
            u[r][i][j] = fmaf(al, cv[i][j], u[r][i][j]);
            ss[r] = fmaf(u[r][i][j], u[r][i][j], ss[r]);
          }
        }
      }
      for (int v = threadIdx.x + kMaxV * kEpThreads; v < nv; v += kEpThreads) {
        float y[kEpVec], c8[kEpVec];
        ld8_f<DT>(Y, (row0 + r) * (int64_t)Dc + (int64_t)v * kEpVec, y);
        ld8_f<DT_F32>(cp, (int64_t)v * kEpVec, c8);
#pragma unroll
        for (int j = 0; j < kEpVec; ++j) {
          const float t = fmaf(al, c8[j], y[j]);
          ss[r] = fmaf(t, t, ss[r]);
        }
      }
    }
  }
  // workgroup sums of squares, all rows at once
#pragma unroll
  for (int r = 0; r < kEpRows; ++r) {
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) ss[r] += __shfl_xor(ss[r], m);
    if (lane_id() == 0) red[r][wave_id()] = ss[r];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kEpRows; ++r) {
    if (r >= nr) break;
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kEpThreads / kWave; ++i) tot += red[r][i];
    const float rs = rsqrtf(tot / (float)Dc + eps);
    const int64_t base = (row0 + r) * (int64_t)Dc;
#pragma unroll
    for (int i = 0; i < kMaxV; ++i) {
      const int v = threadIdx.x + i * kEpThreads;
      if (v < nv) {
        float o[kEpVec];
#pragma unroll
        for (int j = 0; j < kEpVec; ++j) o[j] = u[r][i][j] * rs * wv[i][j];
        st8_nt<DT>(out, base + (int64_t)v * kEpVec, o);
      }
    }
    for (int v = threadIdx.x + kMaxV * kEpThreads; v < nv; v += kEpThreads) {
      float y[kEpVec], c8[kEpVec], w8[kEpVec], o[kEpVec];
      ld8_f<DT>(Y, base + (int64_t)v * kEpVec, y);
      ld8_f<DT_F32>(cp, (int64_t)v * kEpVec, c8);
      ld8_f<DT_F32>(weight, (int64_t)v * kEpVec, w8);
#pragma unroll
      for (int j = 0; j < kEpVec; ++j) o[j] = fmaf(al, c8[j], y[j]) * rs * w8[j];
      st8_nt<DT>(out, base + (int64_t)v * kEpVec, o);
    }
  }
}

// c[ch] = mean over the rows of (Y_ref - Y_q)[., ch]. One workgroup per 64
// channels: thread (phase, lane) sums rows phase, phase + 4, ... of channel
// 64 * blockIdx.x + lane in float64, and the four phases are added in order, so
// the result does not depend on scheduling. (A calibration-time reduction.)
template <int DT>
__global__ __launch_bounds__(kEpThreads) void k_mean_correction(const void* __restrict__ Yr,
                                                                const void* __restrict__ Yq,
                                                                float* __restrict__ c,
                                                                int64_t rows, int Dc) {
  constexpr int kPh = kEpThreads / kWave;
  __shared__ double part[kPh][kWave];
  const int lane = threadIdx.x % kWave, ph = threadIdx.x / kWave;
  const int ch = blockIdx.x * kWave + lane;
  double acc = 0.0;
  if (ch < Dc)
    for (int64_t r = ph; r < rows; r += kPh)
      acc += (double)ld_f<DT>(Yr, r * Dc + ch) - (double)ld_f<DT>(Yq, r * Dc + ch);
  part[ph][lane] = acc;
  __syncthreads();
  if (ph == 0 && ch < Dc) {
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < kPh; ++i) t += part[i][lane];
    c[ch] = (float)(t / (double)rows);
  }
}

}  // namespace

hipError_t launch_epilogue(const Dims& d, int dtype, const void* Y, const float* corr, float alpha,
                           const float* weight, float eps, void* out, hipStream_t st) {
  const int64_t rows = d.B * d.L;
  const int Dc = d.H * d.P;
  const dim3 grid((unsigned)((rows + kEpRows - 1) / kEpRows));
  switch (dtype) {
    case DT_F32: hipLaunchKernelGGL(k_epilogue<DT_F32>, grid, dim3(kEpThreads), 0, st, Y, corr, alpha, weight, eps, out, Dc, rows); break;
    case DT_F16: hipLaunchKernelGGL(k_epilogue<DT_F16>, grid, dim3(kEpThreads), 0, st, Y, corr, alpha, weight, eps, out, Dc, rows); break;
    case DT_BF16: hipLaunchKernelGGL(k_epilogue<DT_BF16>, grid, dim3(kEpThreads), 0, st, Y, corr, alpha, weight, eps, out, Dc, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mean_correction(const Dims& d, int dtype, const void* Yr, const void* Yq, float* c,
                                  hipStream_t st) {
  const int64_t rows = d.B * d.L;
  const int Dc = d.H * d.P;
  const dim3 grid((unsigned)((Dc + kWave - 1) / kWave));
  switch (dtype) {
    case DT_F32: hipLaunchKernelGGL(k_mean_correction<DT_F32>, grid, dim3(kEpThreads), 0, st, Yr, Yq, c, rows, Dc); break;
    case DT_F16: hipLaunchKernelGGL(k_mean_correction<DT_F16>, grid, dim3(kEpThreads), 0, st, Yr, Yq, c, rows, Dc); break;
    case DT_BF16: hipLaunchKernelGGL(k_mean_correction<DT_BF16>, grid, dim3(kEpThreads), 0, st, Yr, Yq, c, rows, Dc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ssd
