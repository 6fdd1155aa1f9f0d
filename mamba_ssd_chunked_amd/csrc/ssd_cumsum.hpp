// ChunkCumsum block body, shared by the module kernel and the fused INT8
// path's preparation launch.
#pragma once

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// ChunkCumsum. One block per (chunk k, batch b, group of kCsHeads heads). dt is
// staged in LDS; one thread per head then forms the float64 prefix sums in
// sequence order (the only serial part), and all threads evaluate the float64
// exponentials and write dAcs / LUT_state with coalesced stores. Padded
// positions past L carry dt = 0, which leaves the running sum unchanged.
// ---------------------------------------------------------------------------
constexpr int kCsHeads = 4;

template <int DT>
__device__ __forceinline__ void chunk_cumsum_block(const void* __restrict__ dt,
                                                   const float* __restrict__ A,
                                                   float* __restrict__ dAcs,
                                                   float* __restrict__ lut,
                                                   uint8_t* __restrict__ qdecay, const Dims& d,
                                                   int k, int64_t b, int hblk) {
  __shared__ float sdt[kCsHeads][256 + 1];
  __shared__ double sa[kCsHeads][256 + 1];
  const int h0 = hblk * kCsHeads;
  const int nh = min(kCsHeads, d.H - h0);
  const int l = d.l;
  const int64_t t0 = (int64_t)k * l;
  const int nvalid = (int)min((int64_t)l, d.L - t0);
  // all of a thread's loads are issued before any is used (chunks are at most
  // 256 positions, so at most 4 per thread); out-of-range entries read element 0
  // and are replaced by 0
  const float Aj = A[h0 + min((int)threadIdx.x, nh - 1)];  // the head of threads 0 .. nh - 1
  float v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = (int)threadIdx.x + 256 * u;
    const int j = idx % kCsHeads, s = idx / kCsHeads;
    const bool ok = idx < kCsHeads * l && j < nh && s < nvalid;
    const float x = ld_f<DT>(dt, ok ? (b * d.L + t0 + s) * d.H + h0 + j : 0);
    v[u] = ok ? x : 0.f;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = (int)threadIdx.x + 256 * u;
    if (idx < kCsHeads * l) sdt[idx % kCsHeads][idx / kCsHeads] = v[u];
  }
  __syncthreads();
  if ((int)threadIdx.x < nh) {
    const int j = threadIdx.x;
    const double Ah = (double)Aj;
    double a = 0.0;
    // sequence order is kept; the LDS reads of each block of 16 steps are issued
    // together so only the float64 additions form the dependent chain
    for (int s0 = 0; s0 < l; s0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = sdt[j][s0 + u];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        a += (double)v[u] * Ah;  // the product is exact in float64
        sa[j][s0 + u] = a;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nh * l; idx += 256) {
    const int j = idx / l, s = idx % l;
    const double a = sa[j][s], alast = sa[j][l - 1];
    const int64_t o = ((b * d.H + h0 + j) * d.c + k) * (int64_t)l + s;
    dAcs[o] = (float)a;
    if (lut) lut[o] = (float)((double)sdt[j][s] * exp(alast - a));
    if (qdecay && s == 0)
      qdecay[(b * d.H + h0 + j) * d.c + k] = (uint8_t)fmin(round(exp(alast) * 128.0), 128.0);
  }
}

}  // namespace ssd
