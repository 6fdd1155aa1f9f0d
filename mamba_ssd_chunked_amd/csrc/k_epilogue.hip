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

// Wave-per-row form, for 16-bit rows of 512 * V channels (V <= 12): a
// workgroup of 8 waves keeps the weight and correction vectors in LDS (loaded
// once) and each wave streams whole rows. A wave holds its row in registers as
// loaded (16-bit, 4 V dwords per lane), forms y + alpha c for the sum of
// squares, reduces it within the wave (no workgroup barrier per row), then
// forms y + alpha c again (the same fused multiply-add, so the same value) for
// the normalised write. At about 76 VGPRs three such workgroups share a CU, so
// 24 rows are in flight per CU, which covers more of the HBM latency than the
// workgroup-per-row form. The grid is at most three workgroups per CU; their
// waves take rows r, r + 8 * gridDim.x, ...
constexpr int kEpwWaves = 8;
constexpr int kEpwMaxDc = 512 * 12;

template <int DT, int V>
__global__ __launch_bounds__(kEpwWaves * kWave) void k_epilogue_w(const void* Y,
                                                                   const float* __restrict__ corr,
                                                                   float alpha,
                                                                   const float* __restrict__ weight,
                                                                   float eps, void* out,
                                                                   int64_t rows) {
  static_assert(DT == DT_F16 || DT == DT_BF16, "16-bit rows");
  typedef typename Store<DT>::T T;
  typedef uint32_t v4u_ __attribute__((ext_vector_type(4)));
  constexpr int Dc = 512 * V;
  __shared__ __attribute__((aligned(16))) float s_w[Dc];
  __shared__ __attribute__((aligned(16))) float s_c[Dc];
  const float* const cp = corr ? corr : weight;  // weight stands in with a zero coefficient
  const float al = corr ? alpha : 0.f;
  for (int i = threadIdx.x; i < Dc / 4; i += kEpwWaves * kWave) {
    ((float4*)s_w)[i] = ((const float4*)weight)[i];
    ((float4*)s_c)[i] = ((const float4*)cp)[i];
  }
  __syncthreads();
  const int lane = lane_id();
  const auto elem = [](const v4u_& v, int e) {
    const uint32_t dw = v[e >> 1];
    return Store<DT>::to_f(__builtin_bit_cast(T, (u16)((e & 1) ? (dw >> 16) : (dw & 0xffffu))));
  };
  for (int64_t row = (int64_t)blockIdx.x * kEpwWaves + wave_id(); row < rows;
       row += (int64_t)gridDim.x * kEpwWaves) {
    const int64_t base = row * (int64_t)Dc;
    v4u_ yv[V];
#pragma unroll
    for (int j = 0; j < V; ++j)
      yv[j] = __builtin_nontemporal_load((const v4u_*)((const u16*)Y + base + (int64_t)(lane + kWave * j) * kEpVec));
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float* c8 = s_c + (lane + kWave * j) * kEpVec;
      const float4 c0 = *(const float4*)c8, c1 = *(const float4*)(c8 + 4);
      const float cv[kEpVec] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int e = 0; e < kEpVec; ++e) {
        const float t = fmaf(al, cv[e], elem(yv[j], e));
        ss = fmaf(t, t, ss);
      }
    }
#pragma unroll
    for (int m = kWave / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    const float rs = rsqrtf(ss / (float)Dc + eps);
    // the loaded row and the correction are opaque here, so the second pass
    // recomputes y + alpha c instead of keeping the first pass's 8 V values live
#pragma unroll
    for (int j = 0; j < V; ++j) asm volatile("" : "+v"(yv[j]));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float* c8 = s_c + (lane + kWave * j) * kEpVec;
      const float* w8 = s_w + (lane + kWave * j) * kEpVec;
      const float4 c0 = *(const float4*)c8, c1 = *(const float4*)(c8 + 4);
      const float4 w0 = *(const float4*)w8, w1 = *(const float4*)(w8 + 4);
      const float cv[kEpVec] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
      const float wv[kEpVec] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float o[kEpVec];
#pragma unroll
      for (int e = 0; e < kEpVec; ++e) o[e] = fmaf(al, cv[e], elem(yv[j], e)) * rs * wv[e];
      st8_nt<DT>(out, base + (int64_t)(lane + kWave * j) * kEpVec, o);
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
  if ((dtype == DT_F16 || dtype == DT_BF16) && Dc % 512 == 0 && Dc <= kEpwMaxDc) {
    const int64_t ncu = cu_count() > 0 ? cu_count() : 256;
    const dim3 gw((unsigned)min((rows + kEpwWaves - 1) / kEpwWaves, 3 * ncu));
#define EPW_(DT_, V_) hipLaunchKernelGGL((k_epilogue_w<DT_, V_>), gw, dim3(kEpwWaves * kWave), 0, st, Y, corr, alpha, weight, eps, out, rows)
#define EPW_DT_(DT_)                  \
    switch (Dc / 512) {               \
      case 1: EPW_(DT_, 1); break;     \
      case 2: EPW_(DT_, 2); break;     \
      case 3: EPW_(DT_, 3); break;     \
      case 4: EPW_(DT_, 4); break;     \
      case 5: EPW_(DT_, 5); break;     \
      case 6: EPW_(DT_, 6); break;     \
      case 7: EPW_(DT_, 7); break;     \
      case 8: EPW_(DT_, 8); break;     \
      case 9: EPW_(DT_, 9); break;     \
      case 10: EPW_(DT_, 10); break;   \
      case 11: EPW_(DT_, 11); break;   \
      default: EPW_(DT_, 12); break;   \
    }
    if (dtype == DT_F16) {
      EPW_DT_(DT_F16);
    } else {
      EPW_DT_(DT_BF16);
    }
#undef EPW_DT_
#undef EPW_
    return hipGetLastError();
  }
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
