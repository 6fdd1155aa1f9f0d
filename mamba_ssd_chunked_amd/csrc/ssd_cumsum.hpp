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
// adds its lanes' totals with a cross-lane scan. The test uses the computed sum of
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

// Inclusive scans across the 64 lanes of a wave on DPP moves (no LDS round
// trips): four row shifts within each row of 16 lanes, then the last lane of
// row 0 broadcast into row 1 (and of row 2 into row 3), then the last lane of
// row 1 into rows 2 and 3. A lane the move does not reach reads the identity.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long x = (unsigned long long)__double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)x, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(x >> 32), CTRL, ROWS, 0xf, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
__device__ __forceinline__ double wave_scan_add(double v) {  // the identity 0.0 (+0)
  v += dpp_f64<0x111, 0xf>(v);  // row_shr:1
  v += dpp_f64<0x112, 0xf>(v);  // row_shr:2
  v += dpp_f64<0x114, 0xf>(v);  // row_shr:4
  v += dpp_f64<0x118, 0xf>(v);  // row_shr:8
  v += dpp_f64<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
  v += dpp_f64<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
  return v;
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_min_step(int v) {
  return min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ int wave_scan_min(int v) {
  v = dpp_min_step<0x111, 0xf>(v);
  v = dpp_min_step<0x112, 0xf>(v);
  v = dpp_min_step<0x114, 0xf>(v);
  v = dpp_min_step<0x118, 0xf>(v);
  v = dpp_min_step<0x142, 0xa>(v);
  v = dpp_min_step<0x143, 0xc>(v);
  return v;
}
__device__ __forceinline__ double lane63_f64(double v) {
  const unsigned long long x = (unsigned long long)__double_as_longlong(v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)x, 63);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(x >> 32), 63);
  return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
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
  // wave totals (the last lane of the inclusive scans)
  sabs = lane63_f64(wave_scan_add(sabs));
  elo = __builtin_amdgcn_readlane(wave_scan_min(elo), 63);
  // (NaN compares false, so inf / NaN products take the chain)
  const bool exact = elo == INT_MAX || sabs < ldexp(1.0, 52 + elo);
  if (exact) {
    const double incl = wave_scan_add(tot);  // inclusive scan of the lane totals
    const double excl = incl - tot;          // exact: a partial sum, see above
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
  const double alast = lane63_f64(R == 4 ? q[3] : (R == 2 ? q[1] : q[0]));  // a at s = l - 1
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
