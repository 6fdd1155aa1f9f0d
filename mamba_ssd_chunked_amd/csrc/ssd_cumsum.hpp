// ChunkCumsum block body, shared by the module kernel and the fused INT8
// path's preparation launch.
#pragma once

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// ChunkCumsum. One block of kCsThreads threads per (chunk k, batch b, group of
// kCsHeads heads). All threads stage dt in LDS with coalesced loads; then wave
// j forms head j's float64 prefix sums a_s of the products dt_s * A (each exact
// in float64), lane i holding the R = l / 64 consecutive positions R i .. R i +
// R - 1, and writes dAcs, LUT_state and Q(Decay) from registers.
//
// The result must equal the float64 additions in sequence order bit for bit.
// Every product is an integer multiple of 2^e, e the exponent of the lowest set
// bit over the chunk's nonzero products, and every partial sum, whatever the
// grouping, is a multiple of 2^e of magnitude at most sum |p_s|. When that bound
// is below 2^(53 + e), every such sum is representable, so each addition is
// exact and any order of summation gives the sequential result: the wave then
// adds its lanes' totals with a shuffle scan. The test uses the computed sum of
// |p_s| against 2^(52 + e), a factor of two that covers its own rounding. For
// heads that fail it (very wide exponent spreads, or inf / NaN), lane 0 runs
// the sequential chain. Padded positions past L carry dt = 0, which leaves the
// running sum unchanged and does not enter e.
// ---------------------------------------------------------------------------
constexpr int kCsHeads = 16;
constexpr int kCsThreads = 1024;
static_assert(kCsThreads == 64 * kCsHeads, "one wave per head");

// exponent of the lowest set bit of a nonzero float64 (p = m 2^(E - 1075), m
// the 53-bit significand; the products here are never subnormal in float64)
__device__ __forceinline__ int cs_lsb_exp(double p) {
  const uint64_t bits = (uint64_t)__double_as_longlong(p);
  const int E = (int)((bits >> 52) & 0x7ff);
  const uint64_t m = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  return E - 1075 + (int)__builtin_ctzll(m);
}

// LDS the block body needs (the caller provides it, so that launches holding
// other block kinds can share one allocation).
struct CsLds {
  float sdt[kCsHeads][256 + 1];
  double sa[kCsHeads][256];  // the sequential chain's prefixes (fallback only)
};

template <int DT>
__device__ __forceinline__ void chunk_cumsum_block(const void* __restrict__ dt,
                                                   const float* __restrict__ A,
                                                   float* __restrict__ dAcs,
                                                   float* __restrict__ lut,
                                                   uint8_t* __restrict__ qdecay, const Dims& d,
                                                   int k, int64_t b, int hblk, CsLds& cs) {
  constexpr int kPer = kCsHeads * 256 / kCsThreads;  // staged entries per thread (chunks <= 256)
  float(&sdt)[kCsHeads][256 + 1] = cs.sdt;
  double(&sa)[kCsHeads][256] = cs.sa;
  const int h0 = hblk * kCsHeads;
  const int nh = min(kCsHeads, d.H - h0);
  const int l = d.l;
  const int64_t t0 = (int64_t)k * l;
  const int nvalid = (int)min((int64_t)l, d.L - t0);
  {
    // entry idx = tid + kCsThreads u is (head idx % kCsHeads, position idx /
    // kCsHeads). All loads of a thread are issued before any is used;
    // out-of-range entries read element 0 and are replaced by 0.
    const int jt = (int)threadIdx.x % kCsHeads;
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
      if (idx < kCsHeads * l) sdt[jt][idx / kCsHeads] = v[u];
    }
  }
  __syncthreads();
  const int j = (int)threadIdx.x / 64, lane = (int)threadIdx.x % 64;
  if (j >= nh) return;  // (wave-uniform; no barrier follows)
  const double Aj = (double)A[h0 + j];
  const int R = l / 64;  // positions per lane: 1, 2 or 4
  float dtv[4];
  double q[4];  // the lane's own inclusive prefixes
  double tot = 0.0, sabs = 0.0;
  int elo = INT_MAX;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    dtv[u] = 0.f;
    q[u] = 0.0;
    if (u < R) {
      dtv[u] = sdt[j][R * lane + u];
      const double p = (double)dtv[u] * Aj;  // exact in float64
      tot += p;
      q[u] = tot;
      sabs += fabs(p);
      if (p != 0.0) elo = min(elo, cs_lsb_exp(p));
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    sabs += __shfl_xor(sabs, m);
    elo = min(elo, __shfl_xor(elo, m));
  }
  // (NaN compares false, so inf / NaN products take the chain)
  const bool exact = elo == INT_MAX || sabs < ldexp(1.0, 52 + elo);
  if (exact) {
    double incl = tot;  // inclusive scan of the lane totals
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const double o = __shfl_up(incl, m);
      if (lane >= m) incl += o;
    }
    const double excl = incl - tot;  // exact: a partial sum, see above
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] += excl;
  } else {
    if (lane == 0) {
      // the LDS reads of each block of 16 steps are issued together, so only the
      // float64 additions form the dependent chain
      double a = 0.0;
      for (int s0 = 0; s0 < l; s0 += 16) {
        float pv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) pv[u] = sdt[j][s0 + u];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          a += (double)pv[u] * Aj;
          sa[j][s0 + u] = a;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u < R) q[u] = sa[j][R * lane + u];
  }
  const double alast = __shfl(R == 4 ? q[3] : (R == 2 ? q[1] : q[0]), 63);  // a at s = l - 1
  const int64_t o0 = ((b * d.H + h0 + j) * d.c + k) * (int64_t)l + R * lane;
  float da[4], lu[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    da[u] = (float)q[u];
    lu[u] = u < R ? (float)((double)dtv[u] * exp(alast - q[u])) : 0.f;
  }
  if (R == 4) {
    *(float4*)(dAcs + o0) = make_float4(da[0], da[1], da[2], da[3]);
    if (lut) *(float4*)(lut + o0) = make_float4(lu[0], lu[1], lu[2], lu[3]);
  } else if (R == 2) {
    *(float2*)(dAcs + o0) = make_float2(da[0], da[1]);
    if (lut) *(float2*)(lut + o0) = make_float2(lu[0], lu[1]);
  } else {
    dAcs[o0] = da[0];
    if (lut) lut[o0] = lu[0];
  }
  if (qdecay && lane == 0)
    qdecay[(b * d.H + h0 + j) * d.c + k] = (uint8_t)fmin(round(exp(alast) * 128.0), 128.0);
}

}  // namespace ssd
