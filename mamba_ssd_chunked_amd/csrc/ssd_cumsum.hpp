// ChunkCumsum block body, shared by the module kernel and the fused INT8
// path's preparation launch.
#pragma once

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// ChunkCumsum. One block of kCsThreads threads per (chunk k, batch b, group of
// kCsHeads heads). All threads stage dt and the products dt * A (exact in
// float64) in LDS; one thread per head then forms the float64 prefix sums in
// sequence order, the only serial part, whose length is set by the latency of
// the dependent float64 additions. The heads' chains sit in the lanes of one
// wave, so few such waves share a SIMD. Finally all threads evaluate the
// float64 exponentials and write dAcs / LUT_state with coalesced stores.
// Padded positions past L carry dt = 0, which leaves the running sum unchanged.
// ---------------------------------------------------------------------------
constexpr int kCsHeads = 16;
constexpr int kCsThreads = 1024;

template <int DT>
__device__ __forceinline__ void chunk_cumsum_block(const void* __restrict__ dt,
                                                   const float* __restrict__ A,
                                                   float* __restrict__ dAcs,
                                                   float* __restrict__ lut,
                                                   uint8_t* __restrict__ qdecay, const Dims& d,
                                                   int k, int64_t b, int hblk) {
  constexpr int kPer = kCsHeads * 256 / kCsThreads;  // staged entries per thread (chunks <= 256)
  __shared__ float sdt[kCsHeads][256 + 1];
  __shared__ double sa[kCsHeads][256 + 1];
  const int h0 = hblk * kCsHeads;
  const int nh = min(kCsHeads, d.H - h0);
  const int l = d.l;
  const int64_t t0 = (int64_t)k * l;
  const int nvalid = (int)min((int64_t)l, d.L - t0);
  // entry idx = tid + kCsThreads u is (head idx % kCsHeads, position idx /
  // kCsHeads), so every entry of a thread belongs to the same head. All loads of
  // a thread are issued before any is used; out-of-range entries read element 0
  // and are replaced by 0.
  const int jt = (int)threadIdx.x % kCsHeads;
  const double Aj = (double)A[h0 + min(jt, nh - 1)];
  float v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int idx = (int)threadIdx.x + kCsThreads * u;
    const int s = idx / kCsHeads;
    const bool ok = idx < kCsHeads * l && jt < nh && s < nvalid;
    const float x = ld_f<DT>(dt, ok ? (b * d.L + t0 + s) * d.H + h0 + jt : 0);
    v[u] = ok ? x : 0.f;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int idx = (int)threadIdx.x + kCsThreads * u;
    if (idx < kCsHeads * l) {
      sdt[jt][idx / kCsHeads] = v[u];
      sa[jt][idx / kCsHeads] = (double)v[u] * Aj;  // the product is exact in float64
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < nh) {
    const int j = threadIdx.x;
    double a = 0.0;
    // sequence order is kept; the LDS reads of each block of 16 steps are issued
    // together so only the float64 additions form the dependent chain
    for (int s0 = 0; s0 < l; s0 += 16) {
      double p[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) p[u] = sa[j][s0 + u];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        a += p[u];
        sa[j][s0 + u] = a;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nh * l; idx += kCsThreads) {
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
