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
// reduce over the R lanes of a row with LDS swizzles (no LDS traffic).
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

// LDS of one wave: per-position vectors of its head.
template <int P, int NS>
struct DecLds {
  float b[NS];   // INT8: float(Q(B)); FLOAT: B
  float c[NS];   // FLOAT: C
  int8_t qc[NS]; // INT8: Q(C)
  float x[P];    // x
  int qx[P];     // INT8: Q(Xs)
};

// ---------------------------------------------------------------------------
// INT8 step
// ---------------------------------------------------------------------------
template <int DT, int P, int NS>
__global__ __launch_bounds__(256) void k_decode_i8(DecodeArgs a) {
  constexpr int R = NS / 16;        // 16-byte slices per state row
  constexpr int RPI = kWave / R;    // rows per wave pass
  constexpr int ITER = (P + RPI - 1) / RPI;
  __shared__ __attribute__((aligned(16))) DecLds<P, NS> lds[kDecWaves];

  const int w = wave_id(), lane = lane_id();
  const int64_t unit = (int64_t)blockIdx.x * kDecWaves + w;
  if (unit >= a.units) return;  // uniform per wave
  DecLds<P, NS>& L = lds[w];
  const int64_t b = unit / a.H;
  const int h = (int)(unit % a.H);
  const int g = h / a.hpg;

  const float dtv = ld_f<DT>(a.dt, unit);
  const float Ah = a.A[h];
  // Q(Decay): the product dt A is exact in float64, the decision is taken there
  const int qd = (int)fmin(round(exp((double)dtv * (double)Ah) * 128.0), 128.0);
  const float decay = __expf(dtv * Ah);

  // Q(B), Q(C) of this position and group; Q(Xs) of this head
  const float ib = a.sc.inv_B[g], ic = a.sc.inv_C[g];
  int cbp = 0;
  for (int n = lane; n < NS; n += kWave) {
    const int64_t o = (b * a.G + g) * NS + n;
    const int qb = q8(__fmul_rn(ld_f<DT>(a.B, o), ib));
    const int qc = q8(__fmul_rn(ld_f<DT>(a.C, o), ic));
    L.b[n] = (float)qb;
    L.qc[n] = (int8_t)qc;
    cbp += qb * qc;
  }
  for (int p = lane; p < P; p += kWave) {
    const float xv = ld_f<DT>(a.X, unit * P + p);
    L.x[p] = xv;
    L.qx[p] = q8(__fmul_rn(__fmul_rn(dtv, xv), a.sc.inv_X[h * P + p]));
  }
  int cb = lane_sum_i<32>(cbp);
  cb += __shfl_xor(cb, 32);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int col = lane % R, r0 = lane / R;
  float fb[16];
#pragma unroll
  for (int e = 0; e < 16; e += 4) {
    const float4 v = *(const float4*)&L.b[16 * col + e];
    fb[e] = v.x; fb[e + 1] = v.y; fb[e + 2] = v.z; fb[e + 3] = v.w;
  }
  const uint4 qcv = *(const uint4*)&L.qc[16 * col];
  const uint32_t qcw[4] = {qcv.x, qcv.y, qcv.z, qcv.w};

  uint4* st = (uint4*)((int8_t*)a.state + unit * (int64_t)P * NS);
  uint4 hv[ITER];
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int row = r0 + i * RPI;
    if (row < P) hv[i] = st[row * R + col];
  }
  const float sC = a.sc.s_C[g];
  const float ydiag = (float)cb * sC * a.sc.s_B[g] * dtv;
  const float Dh = a.D[h];
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int row = r0 + i * RPI;
    const bool ok = row < P;
    const int rr = ok ? row : 0;
    const float fqx = (float)L.qx[rr];
    const float M = a.sc.M_req[h * P + rr];
    const uint32_t hw[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
    uint32_t nw[4];
    int acc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s8 = q8(__fmul_rn(__fmul_rn(fqx, fb[4 * j + e]), M));
        o[e] = sat127(s8 + rsh7_fast(__mul24(qd, byte_s(hw[j], e))));
      }
      nw[j] = perm_pack4(o[0], o[1], o[2], o[3]);
      acc = __builtin_amdgcn_sdot4((int)qcw[j], (int)hw[j], acc, false);
    }
    if (ok) st[row * R + col] = make_uint4(nw[0], nw[1], nw[2], nw[3]);
    acc = lane_sum_i<R>(acc);
    if (ok && col == 0) {
      const float xv = L.x[row];
      const float y = (float)acc * (decay * sC * a.sc.s_S[h * P + row]) + ydiag * xv + Dh * xv;
      ((typename Store<DT>::T*)a.Y)[unit * P + row] = to_store<DT>(y);
    }
  }
}

// ---------------------------------------------------------------------------
// FLOAT step (fp32 state)
// ---------------------------------------------------------------------------
template <int DT, int P, int NS>
__global__ __launch_bounds__(256) void k_decode_f(DecodeArgs a) {
  constexpr int R = NS / 4;         // float4 slices per state row
  constexpr int RPI = kWave / R;
  constexpr int ITER = (P + RPI - 1) / RPI;
  constexpr int KB = ITER < 8 ? ITER : 8;  // rows in flight per lane
  __shared__ __attribute__((aligned(16))) DecLds<P, NS> lds[kDecWaves];

  const int w = wave_id(), lane = lane_id();
  const int64_t unit = (int64_t)blockIdx.x * kDecWaves + w;
  if (unit >= a.units) return;
  DecLds<P, NS>& L = lds[w];
  const int64_t b = unit / a.H;
  const int h = (int)(unit % a.H);
  const int g = h / a.hpg;

  const float dtv = ld_f<DT>(a.dt, unit);
  const float decay = __expf(dtv * a.A[h]);
  for (int n = lane; n < NS; n += kWave) {
    const int64_t o = (b * a.G + g) * NS + n;
    L.b[n] = ld_f<DT>(a.B, o);
    L.c[n] = ld_f<DT>(a.C, o);
  }
  for (int p = lane; p < P; p += kWave) L.x[p] = ld_f<DT>(a.X, unit * P + p);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  const int col = lane % R, r0 = lane / R;
  const float4 bv = *(const float4*)&L.b[4 * col];
  const float4 cv = *(const float4*)&L.c[4 * col];
  const float Dh = a.D[h];
  float4* st = (float4*)((float*)a.state + unit * (int64_t)P * NS);
#pragma unroll
  for (int i0 = 0; i0 < ITER; i0 += KB) {
    float4 hv[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      const int row = r0 + (i0 + j) * RPI;
      if (i0 + j < ITER && row < P) hv[j] = st[row * R + col];
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (i0 + j >= ITER) break;
      const int row = r0 + (i0 + j) * RPI;
      const bool ok = row < P;
      const float xv = L.x[ok ? row : 0];
      const float dx = dtv * xv;
      float4 n;
      n.x = fmaf(decay, hv[j].x, dx * bv.x);
      n.y = fmaf(decay, hv[j].y, dx * bv.y);
      n.z = fmaf(decay, hv[j].z, dx * bv.z);
      n.w = fmaf(decay, hv[j].w, dx * bv.w);
      if (ok) st[row * R + col] = n;
      float acc = cv.x * n.x + cv.y * n.y + cv.z * n.z + cv.w * n.w;
      acc = lane_sum_f<R>(acc);
      if (ok && col == 0)
        ((typename Store<DT>::T*)a.Y)[unit * P + row] = to_store<DT>(acc + Dh * xv);
    }
  }
}

template <int DT, int P, int NS>
hipError_t launch_dec(bool int8, const DecodeArgs& a, hipStream_t st) {
  const int64_t blocks = (a.units + kDecWaves - 1) / kDecWaves;
  if (int8)
    hipLaunchKernelGGL((k_decode_i8<DT, P, NS>), dim3((unsigned)blocks), dim3(kDecWaves * kWave), 0,
                       st, a);
  else
    hipLaunchKernelGGL((k_decode_f<DT, P, NS>), dim3((unsigned)blocks), dim3(kDecWaves * kWave), 0,
                       st, a);
  return hipGetLastError();
}

template <int DT, int P>
hipError_t dispatch_n(bool int8, int N, const DecodeArgs& a, hipStream_t st) {
  switch (N) {
    case 16: return launch_dec<DT, P, 16>(int8, a, st);
    case 32: return launch_dec<DT, P, 32>(int8, a, st);
    case 64: return launch_dec<DT, P, 64>(int8, a, st);
    case 128: return launch_dec<DT, P, 128>(int8, a, st);
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
