// Single-token decode step: the recurrent form of the SSD block, one position
// per call, on the state a forward (or an earlier step) left behind.
//
// FLOAT: h' = exp(dt A) h + dt x (x) B,   y = C . h' + D x        (fp32 state)
// INT8 ("SSDi8" notes page, "Key design 2", Eq. 6, with a chunk of one
// position): Q(Decay) = min(128, RHAZ(128 exp(dt A))) decided in float64;
//   Q(Xs) = sat(RHAZ(fl32(fl32(dt x) inv_X)));  S8 = sat(RHAZ(fl32(Q(Xs) Q(B) M_req)));
//   h' = sat(S8 + RSH7(Q(Decay) h));
//   y = exp(dt A) s_C s_S (Q(C) . h) + (Q(C) . Q(B)) s_C s_B dt x + D x
// (ChunkScan1 reads the state before the step; ChunkScan2 is the single
// diagonal term of the one-position chunk).
//
// One wave per (batch, head), four per workgroup. The state of a head is P
// rows of N values; lane L owns the 16-byte column slice L % R of rows
// L / R + i * (64 / R), R = 16-byte slices per row, so every load and store
// instruction of the wave covers contiguous memory. The row sums of C . h
// reduce over the R lanes of a row with LDS swizzles (no LDS traffic). The
// state is touched once per step, so its loads and stores carry the
// non-temporal hint (streaming past the caches measured faster on the
// in-place read-then-write pattern).
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {
namespace {

constexpr int kDecWaves = 4;

struct DecodeArgs {
  const void* X;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  ScalePtrs sc;
  void* state;
  void* Y;
  int64_t units;  // batch * heads
  int H, G, hpg;
};

// Value of lane (L xor M) within each group of 32 lanes (ds_swizzle bit mode).
template <int M>
__device__ __forceinline__ int swz(int v) {
  return __builtin_amdgcn_ds_swizzle(v, (M << 10) | 0x1f);
}

// Sum over aligned groups of R consecutive lanes (R a power of two <= 32).
template <int R>
__device__ __forceinline__ int lane_sum_i(int v) {
  if constexpr (R >= 2) v += swz<1>(v);
  if constexpr (R >= 4) v += swz<2>(v);
  if constexpr (R >= 8) v += swz<4>(v);
  if constexpr (R >= 16) v += swz<8>(v);
  if constexpr (R >= 32) v += swz<16>(v);
  return v;
}
template <int R>
__device__ __forceinline__ float lane_sum_f(float v) {
  if constexpr (R >= 2) v += __int_as_float(swz<1>(__float_as_int(v)));
  if constexpr (R >= 4) v += __int_as_float(swz<2>(__float_as_int(v)));
  if constexpr (R >= 8) v += __int_as_float(swz<4>(__float_as_int(v)));
  if constexpr (R >= 16) v += __int_as_float(swz<8>(__float_as_int(v)));
  if constexpr (R >= 32) v += __int_as_float(swz<16>(__float_as_int(v)));
  return v;
}

// Low bytes of a, b, c, d packed into one dword (three byte permutes).
__device__ __forceinline__ uint32_t perm_pack4(int a, int b, int c, int d) {
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// LDS of one wave: the per-position vectors of its head.
template <int P, int NS>
struct DecLdsI8 {
  float b[NS];     // float(Q(B))
  int8_t qc[NS];   // Q(C)
  float4 rv[P];    // per state row p: float(Q(Xs)), M_req, x, exp(dt A) s_C s_S
};
template <int P, int NS>
struct DecLdsF {
  float b[NS];     // B
  float c[NS];     // C
  float x[P];      // x
};

// ---------------------------------------------------------------------------
// INT8 step
// ---------------------------------------------------------------------------
template <int DT, int P, int NS, int SPLIT>
__global__ __launch_bounds__(256) void k_decode_i8(DecodeArgs a) {
  constexpr int R = NS / 16;        // 16-byte slices per state row
  constexpr int RPI = kWave / R;    // rows per wave pass
  constexpr int ITER = (P + RPI - 1) / RPI / SPLIT;  // passes of this wave
  __shared__ __attribute__((aligned(16))) DecLdsI8<P, NS> lds[kDecWaves];

  const int w = wave_id(), lane = lane_id();
  const int64_t item = (int64_t)blockIdx.x * kDecWaves + w;
  if (item >= a.units * SPLIT) return;  // uniform per wave
  const int64_t unit = item / SPLIT;
  // the state rows are loaded first: they depend on nothing else
  const int col = lane % R, r0 = lane / R + (int)(item % SPLIT) * ITER * RPI;
  v4u* st = (v4u*)((int8_t*)a.state + unit * (int64_t)P * NS);
  v4u hv[ITER];
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int row = r0 + i * RPI;
    if (row < P) hv[i] = __builtin_nontemporal_load(&st[row * R + col]);
  }
  DecLdsI8<P, NS>& L = lds[w];
  const int64_t b = unit / a.H;
  const int h = (int)(unit % a.H);
  const int g = h / a.hpg;

  // every per-position input is loaded before any of it is used, so the
  // prologue costs one memory round trip
  constexpr int NB = (NS + kWave - 1) / kWave;
  float bq[NB], cq[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int n = lane + k * kWave;
    const int64_t o = (b * a.G + g) * NS + n;
    bq[k] = n < NS ? ld_f<DT>(a.B, o) : 0.f;
    cq[k] = n < NS ? ld_f<DT>(a.C, o) : 0.f;
  }
  const bool pl = lane < P;  // P <= 64: one state row per lane
  const int hp = h * P + (pl ? lane : 0);
  const float xv = pl ? ld_f<DT>(a.X, unit * P + lane) : 0.f;
  const float ixv = a.sc.inv_X[hp], mv = a.sc.M_req[hp], ssv = a.sc.s_S[hp];
  const float dtv = ld_f<DT>(a.dt, unit);
  const float Ah = a.A[h];
  const float ib = a.sc.inv_B[g], ic = a.sc.inv_C[g], sC = a.sc.s_C[g];

  // Q(Decay): the product dt A is exact in float64, the decision is taken there
  const int qd = (int)fmin(round(exp((double)dtv * (double)Ah) * 128.0), 128.0);
  const float decay = __expf(dtv * Ah);

  // Q(B), Q(C) of this position and group; Q(Xs) of this head
  int cbp = 0;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int n = lane + k * kWave;
    const int qb = q8(__fmul_rn(bq[k], ib));
    const int qc = q8(__fmul_rn(cq[k], ic));
    if (n < NS) {
      L.b[n] = (float)qb;
      L.qc[n] = (int8_t)qc;
      cbp += qb * qc;
    }
  }
  if (pl) {
    const int qx = q8(__fmul_rn(__fmul_rn(dtv, xv), ixv));
    L.rv[lane] = make_float4((float)qx, mv, xv, decay * sC * ssv);
  }
  int cb = lane_sum_i<32>(cbp);
  cb += __shfl_xor(cb, 32);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  float fb[16];
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 v = *(const float4*)&L.b[16 * col + e];
    fb[e] = v.x; fb[e + 1] = v.y; fb[e + 2] = v.z; fb[e + 3] = v.w;
  }
  const uint4 qcv = *(const uint4*)&L.qc[16 * col];
  const uint32_t qcw[4] = {qcv.x, qcv.y, qcv.z, qcv.w};

  const float ydiag = (float)cb * sC * a.sc.s_B[g] * dtv;
  const float Dh = a.D[h];
  const v2s qd2 = {(short)qd, (short)qd};
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int row = r0 + i * RPI;
    const bool ok = row < P;
    const int rr = ok ? row : 0;
    const float4 rv = L.rv[rr];
    const float fqx = rv.x, M = rv.y;
    const uint32_t hw[4] = {hv[i][0], hv[i][1], hv[i][2], hv[i][3]};
    uint32_t nw[4];
    int acc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float c[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = q8_pre(__fmul_rn(__fmul_rn(fqx, fb[4 * j + e]), M));
      const v2s s01 = cvt_pair(c[0], c[1]), s23 = cvt_pair(c[2], c[3]);
      const v2s r01 = rsh7_pair(qd2, unpack_pair(hw[j], 0x010c000cu));
      const v2s r23 = rsh7_pair(qd2, unpack_pair(hw[j], 0x030c020cu));
      nw[j] = pack_pairs(sat127_pair(s01 + r01), sat127_pair(s23 + r23));
      acc = __builtin_amdgcn_sdot4((int)qcw[j], (int)hw[j], acc, false);
    }
    if (ok) __builtin_nontemporal_store((v4u){nw[0], nw[1], nw[2], nw[3]}, &st[row * R + col]);
    acc = lane_sum_i<R>(acc);
    if (ok && col == 0) {
      const float y = (float)acc * rv.w + ydiag * rv.z + Dh * rv.z;
      ((typename Store<DT>::T*)a.Y)[unit * P + row] = to_store<DT>(y);
    }
  }
}

// ---------------------------------------------------------------------------
// FLOAT step (fp32 state)
// ---------------------------------------------------------------------------
template <int DT, int P, int NS, int SPLIT>
__global__ __launch_bounds__(256) void k_decode_f(DecodeArgs a) {
  constexpr int R = NS / 4;         // float4 slices per state row
  constexpr int RPI = kWave / R;
  constexpr int ITER = (P + RPI - 1) / RPI / SPLIT;
  constexpr int KB = ITER < 8 ? ITER : 8;  // rows in flight per lane
  __shared__ __attribute__((aligned(16))) DecLdsF<P, NS> lds[kDecWaves];

  const int w = wave_id(), lane = lane_id();
  const int64_t item = (int64_t)blockIdx.x * kDecWaves + w;
  if (item >= a.units * SPLIT) return;
  const int64_t unit = item / SPLIT;
  // rows are processed in batches of KB per lane; the next batch's loads are
  // issued before the current batch is updated, the first before the prologue
  const int col = lane % R, r0 = lane / R + (int)(item % SPLIT) * ITER * RPI;
  v4f* st = (v4f*)((float*)a.state + unit * (int64_t)P * NS);
  auto load_batch = [&](int i0, v4f* hv) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int row = r0 + (i0 + j) * RPI;
      if (i0 + j < ITER && row < P) hv[j] = __builtin_nontemporal_load(&st[row * R + col]);
    }
  };
  v4f cur[KB];
  load_batch(0, cur);
  DecLdsF<P, NS>& L = lds[w];
  const int64_t b = unit / a.H;
  const int h = (int)(unit % a.H);
  const int g = h / a.hpg;

  constexpr int NB = (NS + kWave - 1) / kWave;
  float bq[NB], cq[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int n = lane + k * kWave;
    const int64_t o = (b * a.G + g) * NS + n;
    bq[k] = n < NS ? ld_f<DT>(a.B, o) : 0.f;
    cq[k] = n < NS ? ld_f<DT>(a.C, o) : 0.f;
  }
  const float xv0 = lane < P ? ld_f<DT>(a.X, unit * P + lane) : 0.f;  // P <= 64
  const float dtv = ld_f<DT>(a.dt, unit);
  const float decay = __expf(dtv * a.A[h]);
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int n = lane + k * kWave;
    if (n < NS) {
      L.b[n] = bq[k];
      L.c[n] = cq[k];
    }
  }
  if (lane < P) L.x[lane] = xv0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const float4 bv = *(const float4*)&L.b[4 * col];
  const float4 cv = *(const float4*)&L.c[4 * col];
  const float Dh = a.D[h];
#pragma unroll
  for (int i0 = 0; i0 < ITER; i0 += KB) {
    v4f nxt[KB];
    if (i0 + KB < ITER) load_batch(i0 + KB, nxt);
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (i0 + j >= ITER) break;
      const int row = r0 + (i0 + j) * RPI;
      const bool ok = row < P;
      const float xv = L.x[ok ? row : 0];
      const float dx = dtv * xv;
      v4f n;
      n[0] = fmaf(decay, cur[j][0], dx * bv.x);
      n[1] = fmaf(decay, cur[j][1], dx * bv.y);
      n[2] = fmaf(decay, cur[j][2], dx * bv.z);
      n[3] = fmaf(decay, cur[j][3], dx * bv.w);
      if (ok) __builtin_nontemporal_store(n, &st[row * R + col]);
      float acc = cv.x * n[0] + cv.y * n[1] + cv.z * n[2] + cv.w * n[3];
      acc = lane_sum_f<R>(acc);
      if (ok && col == 0)
        ((typename Store<DT>::T*)a.Y)[unit * P + row] = to_store<DT>(acc + Dh * xv);
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) cur[j] = nxt[j];
  }
}

template <bool I8, int DT, int P, int NS, int SPLIT>
hipError_t launch_dec_s(const DecodeArgs& a, hipStream_t st) {
  const int64_t blocks = (a.units * SPLIT + kDecWaves - 1) / kDecWaves;
  if constexpr (I8)
    hipLaunchKernelGGL((k_decode_i8<DT, P, NS, SPLIT>), dim3((unsigned)blocks),
                       dim3(kDecWaves * kWave), 0, st, a);
  else
    hipLaunchKernelGGL((k_decode_f<DT, P, NS, SPLIT>), dim3((unsigned)blocks),
                       dim3(kDecWaves * kWave), 0, st, a);
  return hipGetLastError();
}

// A head's rows are split over SPLIT = 4 waves when one wave per head would
// leave the chip short of waves (fewer than 16 per CU): a small batch is
// latency-bound, and four shorter waves finish sooner than one long one. Each
// wave still forms the whole head's per-position vectors.
template <bool I8, int DT, int P, int NS>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t st) {
  constexpr int RPI = kWave / (NS / (I8 ? 16 : 4));  // rows per wave pass
  constexpr int ITER = (P + RPI - 1) / RPI;          // passes of one wave per head
  if constexpr (ITER % 4 == 0) {
    const int64_t ncu = cu_count();
    if (a.units * 4 <= 16 * (ncu > 0 ? ncu : 256)) return launch_dec_s<I8, DT, P, NS, 4>(a, st);
  }
  return launch_dec_s<I8, DT, P, NS, 1>(a, st);
}

template <int DT, int P>
hipError_t dispatch_n(bool int8, int N, const DecodeArgs& a, hipStream_t st) {
  switch (N) {
    case 16: return int8 ? launch_dec<true, DT, P, 16>(a, st) : launch_dec<false, DT, P, 16>(a, st);
    case 32: return int8 ? launch_dec<true, DT, P, 32>(a, st) : launch_dec<false, DT, P, 32>(a, st);
    case 64: return int8 ? launch_dec<true, DT, P, 64>(a, st) : launch_dec<false, DT, P, 64>(a, st);
    case 128: return int8 ? launch_dec<true, DT, P, 128>(a, st) : launch_dec<false, DT, P, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int DT>
hipError_t dispatch_p(bool int8, int P, int N, const DecodeArgs& a, hipStream_t st) {
  switch (P) {
    case 16: return dispatch_n<DT, 16>(int8, N, a, st);
    case 32: return dispatch_n<DT, 32>(int8, N, a, st);
    case 64: return dispatch_n<DT, 64>(int8, N, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_step(const Dims& d, int dtype, bool int8, const void* X, const void* dt,
                              const float* A, const void* B, const void* C, const float* D,
                              const ScalePtrs& sc, void* state, void* Y, hipStream_t st) {
  DecodeArgs a{X, dt, A, B, C, D, sc, state, Y, d.B * (int64_t)d.H, d.H, d.G, d.hpg};
  switch (dtype) {
    case DT_F32: return dispatch_p<DT_F32>(int8, d.P, d.N, a, st);
    case DT_F16: return dispatch_p<DT_F16>(int8, d.P, d.N, a, st);
    case DT_BF16: return dispatch_p<DT_BF16>(int8, d.P, d.N, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ssd
