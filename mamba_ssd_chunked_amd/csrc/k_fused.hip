// Fused SSD forward on the persistent-INT8 path ("SSDi8" notes page, "Overall
// framework" and "Key designs 1-3").
//
// Two prologue launches quantise B and C once per group (also writing Q(B)
// transposed per chunk) and form the float64 in-chunk cumulative sums. The main
// kernel then runs one workgroup (four waves) per (batch, head). It walks the
// chunks in order and keeps that head's INT8 state in registers, so the state
// never travels through HBM:
//
//   ChunkState   S32^T[n,p] = sum_s Q(B)^T[n,s] Q(Xs)[s,p]   (int8 MFMA; wave w
//                owns p-tile w), requantised in registers to S8;
//   ChunkScan1   Y_off[s,p] = sum_n Q(C)[s,n] H8_{k-1}[p,n]  (int8 MFMA, H8 from LDS);
//   ChunkBMM     CB^T tiles = Q(B) rows x Q(C) rows          (int8 MFMA; the output
//                lane layout is exactly ChunkScan2's A-operand layout);
//   ChunkScan2   Y_diag = W x, W = CB * s_C s_B * exp(a_s - a_s') dt_s'  (fp16 MFMA);
//   StatePassing H8_k = sat(S8_k + RSH7(Q(Decay_k) H8_{k-1}))  (Eq. 6, in registers).
//
// ChunkScan2 factorisation (exact algebra): for a column tile j strictly below
// row tile i, exp(a_s - a_s') = u_s * V_i[s'] with u_s = exp(a_s - a_{16i}) <= 1
// and V_i[s'] = exp(a_{16i} - a_s') <= 1, so each row tile needs one small table
// V_i and one factor per row instead of an exponential per element. Diagonal
// tiles use exp(a_s - a_s') directly and accumulate separately.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {
namespace {

constexpr int kP = 64;  // head dim handled by the fused kernel (one 16-wide p tile per wave)

__device__ __forceinline__ int rsh7_i(int v) { return rsh7(v); }

// Saturating int8 quantiser with round half away from zero. For |v| <= 127
// after the clamp, trunc(v + copysign(0.5 - 2^-25, v)) equals RHAZ(v) for every
// float32 v (0.5 - 2^-25 keeps 0.5 - 2^-25 itself from rounding up while exact
// ties still reach the next integer); the exhaustive check lives in the tests.
__device__ __forceinline__ int q8(float v) {
  const float c = fminf(fmaxf(v, -127.f), 127.f);
  return (int)(c + __builtin_copysignf(0.49999997f, c));
}

// ---------------------------------------------------------------------------
// Prologue: Q(B), Q(C) with padded rows (t >= L -> 0) and Q(B)^T per chunk.
// grid (c, B*G), 256 threads; one l x N tile per block.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_prologue_bc(Dims d, const void* __restrict__ B,
                                                     const void* __restrict__ C,
                                                     const float* __restrict__ inv_B,
                                                     const float* __restrict__ inv_C,
                                                     int8_t* __restrict__ qB,
                                                     int8_t* __restrict__ qC,
                                                     int8_t* __restrict__ qBT) {
  __shared__ __attribute__((aligned(16))) int8_t tT[128][256 + 16];  // [n][s]
  const int k = blockIdx.x;
  const int64_t bg = blockIdx.y;
  const int64_t b = bg / d.G;
  const int g = (int)(bg % d.G);
  const int N = d.N, l = d.l;
  const int64_t Lp = (int64_t)d.c * l;
  const float ib = inv_B[g], ic = inv_C[g];
  for (int item = threadIdx.x; item < l * (N / 8); item += 256) {
    const int s = item / (N / 8), n0 = (item % (N / 8)) * 8;
    const int64_t t = (int64_t)k * l + s;
    int qb[8], qc[8];
    if (t < d.L) {
      float xb[8], xc[8];
      const int64_t src = ((b * d.L + t) * d.G + g) * (int64_t)N + n0;
      ld8_f<DT>(B, src, xb);
      ld8_f<DT>(C, src, xc);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        qb[j] = q_sat(xb[j] * ib, 127.f);
        qc[j] = q_sat(xc[j] * ic, 127.f);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) qb[j] = qc[j] = 0;
    }
    const int64_t dst = ((b * Lp + t) * d.G + g) * (int64_t)N + n0;
    *(uint2*)(qB + dst) = make_uint2(pack4(qb[0], qb[1], qb[2], qb[3]), pack4(qb[4], qb[5], qb[6], qb[7]));
    *(uint2*)(qC + dst) = make_uint2(pack4(qc[0], qc[1], qc[2], qc[3]), pack4(qc[4], qc[5], qc[6], qc[7]));
#pragma unroll
    for (int j = 0; j < 8; ++j) tT[n0 + j][s] = (int8_t)qb[j];
  }
  __syncthreads();
  // Q(B)^T rows: [b][k][g][n][s], 16 bytes per store
  int8_t* dstT = qBT + ((b * d.c + k) * d.G + g) * (int64_t)N * l;
  for (int item = threadIdx.x; item < N * (l / 16); item += 256) {
    const int n = item / (l / 16), s0 = (item % (l / 16)) * 16;
    *(uint4*)(dstT + (int64_t)n * l + s0) = *(const uint4*)&tT[n][s0];
  }
}

// ---------------------------------------------------------------------------
// main fused kernel
// ---------------------------------------------------------------------------
struct FusedArgs {
  Dims d;
  const void* X;
  const void* dt;
  const int8_t* qB;
  const int8_t* qBT;
  const int8_t* qC;
  const float* dAcs;
  const float* lut;
  const uint8_t* qdecay;
  const float* D;
  ScalePtrs sc;
  void* Y;
  int8_t* final_state;
  int8_t* tap_qxs;
  int32_t* tap_s32;
  int8_t* tap_s8;
  int8_t* tap_passed;
};

// LDS swizzles: XOR the 16-byte chunk index of a row with low row bits so the
// 16 lanes of an MFMA operand read (one row each) spread over the banks.
template <int LC>
__device__ __forceinline__ int xT_off(int p, int s) {  // half index into xT[kP][LC]
  const int ch = (s >> 3) ^ (p & 7);
  return p * LC + ch * 8 + (s & 7);
}
template <int NS>
__device__ __forceinline__ int row_off(int r, int n) {  // byte index into [rows][NS] int8 tiles
  constexpr int nch = NS / 16;
  const int ch = (n >> 4) ^ (r & (nch - 1) & 7);
  return r * NS + ch * 16 + (n & 15);
}

// Eight 2-byte input values (two runs of four) as an MFMA operand fragment.
template <int DT>
__device__ __forceinline__ FragF<DT> frag_from_halves(uint2 lo, uint2 hi) {
  FragF<DT> f;
  const uint32_t w4[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u16 a = (u16)(w4[j] & 0xffff), b2 = (u16)(w4[j] >> 16);
    if constexpr (DT == DT_F16) {
      f.v[2 * j] = __builtin_bit_cast(_Float16, a);
      f.v[2 * j + 1] = __builtin_bit_cast(_Float16, b2);
    } else {
      f.v[2 * j] = __builtin_bit_cast(__bf16, a);
      f.v[2 * j + 1] = __builtin_bit_cast(__bf16, b2);
    }
  }
  return f;
}

template <int DT, int LC, int NS>
__global__ __launch_bounds__(256, 2) void k_fused_i8(FusedArgs a) {
  typedef typename Store<DT>::T T;
  constexpr int RT = LC / 16;  // row tiles of the chunk
  constexpr int NT = NS / 16;  // n tiles of the state
  constexpr int KS = LC / 64;  // ChunkState K steps (64 positions each)
  constexpr int KN = NS / 64;  // K steps over N (64 each)

  __shared__ __attribute__((aligned(16))) T xT[kP * LC];        // x transposed [p][s]
  __shared__ __attribute__((aligned(16))) int8_t qBl[LC * NS];  // Q(B) rows [s][n]
  __shared__ __attribute__((aligned(16))) int8_t H8l[kP * NS];  // passed state [p][n]
  __shared__ __attribute__((aligned(16))) float dAl[LC];
  __shared__ __attribute__((aligned(16))) float dtl[LC];
  __shared__ __attribute__((aligned(16))) float lutl[LC];
  __shared__ __attribute__((aligned(16))) float Vw[4][LC];      // per-wave ChunkScan2 table

  const Dims& d = a.d;
  const int h = blockIdx.x % d.H;
  const int64_t b = blockIdx.x / d.H;
  const int g_h = h / d.hpg;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t Lp = (int64_t)d.c * LC;
  const int H = d.H;

  const int p_own = 16 * w + l16;  // p handled by this lane in ChunkState / StatePassing
  const float invx = a.sc.inv_X[h * kP + p_own];
  const float mreq = a.sc.M_req[h * kP + p_own];
  const float scBC = a.sc.s_C[g_h] * a.sc.s_B[g_h];
  const float sC = a.sc.s_C[g_h];
  const float Dh = a.D[h];
  float sS[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) sS[pt] = a.sc.s_S[h * kP + 16 * pt + l16];

  uint32_t H8[NT];  // passed state, lane (p_own, n = 16 nt + 4 lg + r), 4 int8 per dword
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) H8[nt] = 0;

  for (int k = 0; k < d.c; ++k) {
    const int64_t t0 = (int64_t)k * LC;
    // ---------------- phase A: stage the chunk in LDS ----------------
    // x: thread -> (4 consecutive rows, one 16-byte column chunk); transposed via register shuffles
    for (int item = tid; item < (LC / 4) * (kP / 8); item += 256) {
      const int q = item / (kP / 8), c8 = item % (kP / 8);
      uint4 v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 4 * q + r;
        v[r] = (t < d.L) ? *(const uint4*)((const T*)a.X + ((b * d.L + t) * H + h) * (int64_t)kP + 8 * c8)
                         : make_uint4(0, 0, 0, 0);
      }
      const uint32_t* w0 = (const uint32_t*)&v[0];
      const uint32_t* w1 = (const uint32_t*)&v[1];
      const uint32_t* w2 = (const uint32_t*)&v[2];
      const uint32_t* w3 = (const uint32_t*)&v[3];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // dword e of each row holds p = 8 c8 + 2e (low half) and 2e + 1 (high half)
        const uint32_t lo01 = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(w3[e], w2[e], 0x07060302u);
        const int p0 = 8 * c8 + 2 * e;
        *(uint2*)&xT[xT_off<LC>(p0, 4 * q)] = make_uint2(lo01, lo23);
        *(uint2*)&xT[xT_off<LC>(p0 + 1, 4 * q)] = make_uint2(hi01, hi23);
      }
    }
    // Q(B) rows of the chunk (padded rows are zero in the workspace)
    {
      const int8_t* src = a.qB + ((b * Lp + t0) * d.G + g_h) * (int64_t)NS;
      for (int item = tid; item < LC * (NS / 16); item += 256) {
        const int s = item / (NS / 16), c16 = item % (NS / 16);
        const uint4 v = *(const uint4*)(src + (int64_t)s * d.G * NS + 16 * c16);
        *(uint4*)&qBl[row_off<NS>(s, 16 * c16)] = v;
      }
    }
    for (int s = tid; s < LC; s += 256) {
      const int64_t ci = ((b * H + h) * d.c + k) * (int64_t)LC + s;
      dAl[s] = a.dAcs[ci];
      lutl[s] = a.lut[ci];
      const int64_t t = t0 + s;
      dtl[s] = (t < d.L) ? Store<DT>::to_f(((const T*)a.dt)[(b * d.L + t) * H + h]) : 0.f;
    }
    __syncthreads();

    // ---------------- phase B1: ChunkState^T for p tile w ----------------
    uint32_t S8[NT];
    {
      v4i acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = v4i{0, 0, 0, 0};
      const int8_t* qbt = a.qBT + ((b * d.c + k) * d.G + g_h) * (int64_t)NS * LC;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int s0 = 64 * ks + 16 * lg;
        // Q(Xs) for (p_own, s0 .. s0 + 15)
        const uint4 xa = *(const uint4*)&xT[xT_off<LC>(p_own, s0)];
        const uint4 xb = *(const uint4*)&xT[xT_off<LC>(p_own, s0 + 8)];
        const T* xv0 = (const T*)&xa;
        const T* xv1 = (const T*)&xb;
        int q[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          q[e] = q8((lutl[s0 + e] * Store<DT>::to_f(xv0[e])) * invx);
          q[e + 8] = q8((lutl[s0 + 8 + e] * Store<DT>::to_f(xv1[e])) * invx);
        }
        v4i bq;
#pragma unroll
        for (int j = 0; j < 4; ++j) bq[j] = (int)pack4(q[4 * j], q[4 * j + 1], q[4 * j + 2], q[4 * j + 3]);
        if (a.tap_qxs) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int64_t t = t0 + s0 + e;
            if (t < d.L) a.tap_qxs[((b * d.L + t) * H + h) * (int64_t)kP + p_own] = (int8_t)q[e];
          }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const v4i qa = *(const v4i*)(qbt + (int64_t)(16 * nt + l16) * LC + s0);
          acc[nt] = mma_i8(qa, bq, acc[nt]);
        }
      }
      if (a.tap_s32) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kP + p_own) * NS + 16 * nt + 4 * lg;
          *(int4*)(a.tap_s32 + so) = make_int4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
        }
      }
      // requantise in registers (Key design 2)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        int o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = q8((float)acc[nt][r] * mreq);
        S8[nt] = pack4(o[0], o[1], o[2], o[3]);
      }
    }

    // ---------------- phase B2: ChunkScan for row tiles w, w+4, ... ----------------
#pragma unroll 1
    for (int i = w; i < RT; i += 4) {
      const int s_row = 16 * i + l16;  // A-operand row (and CB^T column) of this lane
      v4i qc[KN];
      {
        const int8_t* src = a.qC + ((b * Lp + t0 + s_row) * d.G + g_h) * (int64_t)NS + 16 * lg;
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) qc[kn] = *(const v4i*)(src + 64 * kn);
      }
      // ChunkScan1 (inter-chunk): int8 state from LDS
      v4i acc1[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc1[pt] = v4i{0, 0, 0, 0};
      if (k > 0) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
          for (int kn = 0; kn < KN; ++kn) {
            const v4i hb = *(const v4i*)&H8l[row_off<NS>(16 * pt + l16, 64 * kn + 16 * lg)];
            acc1[pt] = mma_i8(qc[kn], hb, acc1[pt]);
          }
        }
      }
      // per-wave table V_i[s'] = s_C s_B exp(a_{16i} - a_s') dt_s' for s' < 16 i
      const float a_ref = dAl[16 * i];
      for (int sp = lane; sp < 16 * i; sp += 64) Vw[w][sp] = scBC * __expf(a_ref - dAl[sp]) * dtl[sp];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      v4f acc_off[4], acc_dg[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        acc_off[pt] = v4f{0, 0, 0, 0};
        acc_dg[pt] = v4f{0, 0, 0, 0};
      }
      // off-diagonal column tiles j < i, in pairs (jA, jB)
      for (int jA = 0; jA < i; jA += 2) {
        const int jB = jA + 1;
        const bool hasB = jB < i;
        v4i cbA = v4i{0, 0, 0, 0}, cbB = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          const v4i ba = *(const v4i*)&qBl[row_off<NS>(16 * jA + l16, 64 * kn + 16 * lg)];
          cbA = mma_i8(ba, qc[kn], cbA);
        }
        if (hasB) {
#pragma unroll
          for (int kn = 0; kn < KN; ++kn) {
            const v4i bb = *(const v4i*)&qBl[row_off<NS>(16 * jB + l16, 64 * kn + 16 * lg)];
            cbB = mma_i8(bb, qc[kn], cbB);
          }
        }
        const float4 vA = *(const float4*)&Vw[w][16 * jA + 4 * lg];
        const float4 vB = hasB ? *(const float4*)&Vw[w][16 * jB + 4 * lg] : make_float4(0.f, 0.f, 0.f, 0.f);
        FragF<DT> af;
        af.set(0, (float)cbA[0] * vA.x);
        af.set(1, (float)cbA[1] * vA.y);
        af.set(2, (float)cbA[2] * vA.z);
        af.set(3, (float)cbA[3] * vA.w);
        af.set(4, (float)cbB[0] * vB.x);
        af.set(5, (float)cbB[1] * vB.y);
        af.set(6, (float)cbB[2] * vB.z);
        af.set(7, (float)cbB[3] * vB.w);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const int p = 16 * pt + l16;
          const uint2 xa = *(const uint2*)&xT[xT_off<LC>(p, 16 * jA + 4 * lg)];
          const uint2 xb = hasB ? *(const uint2*)&xT[xT_off<LC>(p, 16 * jB + 4 * lg)] : make_uint2(0, 0);
          acc_off[pt] = FragF<DT>::mma(af, frag_from_halves<DT>(xa, xb), acc_off[pt]);
        }
      }
      // diagonal tile j = i
      {
        v4i cbD = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          const v4i bd = *(const v4i*)&qBl[row_off<NS>(16 * i + l16, 64 * kn + 16 * lg)];
          cbD = mma_i8(bd, qc[kn], cbD);
        }
        const float a_s = dAl[s_row];
        FragF<DT> af;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sp = 16 * i + 4 * lg + r;
          const float wv = (sp <= s_row) ? (float)cbD[r] * scBC * __expf(a_s - dAl[sp]) * dtl[sp] : 0.f;
          af.set(r, wv);
          af.set(r + 4, 0.f);
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const int p = 16 * pt + l16;
          const uint2 xa = *(const uint2*)&xT[xT_off<LC>(p, 16 * i + 4 * lg)];
          acc_dg[pt] = FragF<DT>::mma(af, frag_from_halves<DT>(xa, make_uint2(0, 0)), acc_dg[pt]);
        }
      }
      // epilogue: rows s_out = 16 i + 4 lg + r, columns p = 16 pt + l16
      float u[4], eo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float as = dAl[16 * i + 4 * lg + r];
        u[r] = __expf(as - a_ref);
        eo[r] = __expf(as) * sC;
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int p = 16 * pt + l16;
        const uint2 xr = *(const uint2*)&xT[xT_off<LC>(p, 16 * i + 4 * lg)];
        const T* xv = (const T*)&xr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s_out = 16 * i + 4 * lg + r;
          const int64_t t = t0 + s_out;
          float y = u[r] * acc_off[pt][r] + acc_dg[pt][r] + Dh * Store<DT>::to_f(xv[r]);
          if (k > 0) y += (float)acc1[pt][r] * (eo[r] * sS[pt]);
          if (t < d.L) ((T*)a.Y)[((b * d.L + t) * H + h) * (int64_t)kP + p] = Store<DT>::from_f(y);
        }
      }
      __builtin_amdgcn_wave_barrier();  // Vw reuse by the next row tile
    }
    __syncthreads();

    // ---------------- phase C: StatePassing (Eq. 6) in registers ----------------
    {
      const int qd = a.qdecay[(b * H + h) * d.c + k];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (k == 0) {
          H8[nt] = S8[nt];
        } else {
          int o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int hv = byte_s(S8[nt], r) + rsh7_i(qd * byte_s(H8[nt], r));
            o[r] = hv > 127 ? 127 : (hv < -127 ? -127 : hv);
          }
          H8[nt] = pack4(o[0], o[1], o[2], o[3]);
        }
        // publish for the next chunk's ChunkScan1: H8l[p_own][16 nt + 4 lg .. +3]
        *(uint32_t*)&H8l[row_off<NS>(p_own, 16 * nt + 4 * lg)] = H8[nt];
        const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kP + p_own) * NS + 16 * nt + 4 * lg;
        if (a.tap_s8) *(uint32_t*)(a.tap_s8 + so) = S8[nt];
        if (a.tap_passed) *(uint32_t*)(a.tap_passed + so) = H8[nt];
      }
    }
  }
  if (a.final_state) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t fo = ((b * H + h) * (int64_t)kP + p_own) * NS + 16 * nt + 4 * lg;
      *(uint32_t*)(a.final_state + fo) = H8[nt];
    }
  }
}

constexpr size_t kAl = 256;
size_t al(size_t v) { return (v + kAl - 1) / kAl * kAl; }

}  // namespace

bool fused_supported(const Dims& d, int dtype, bool int8) {
  if (!int8) return false;
  if (d.B * d.G > 65535 || d.B * d.H > (int64_t)1 << 30) return false;
  if (dtype != DT_F16 && dtype != DT_BF16) return false;
  if (d.P != kP) return false;
  if (d.N != 64 && d.N != 128) return false;
  if (d.l != 128 && d.l != 256) return false;
  return true;
}

size_t fused_workspace_bytes(const Dims& d, bool) {
  const size_t Lp = (size_t)d.c * d.l;
  const size_t qbc = (size_t)d.B * Lp * d.G * d.N;
  const size_t cs = (size_t)d.B * d.H * d.c * d.l * sizeof(float);
  const size_t qd = (size_t)d.B * d.H * d.c;
  return 3 * al(qbc) + 2 * al(cs) + al(qd);
}

hipError_t launch_forward_fused(const Dims& d, int dtype, bool int8, const void* X,
                                const void* dt, const float* A, const void* B, const void* C,
                                const float* D, const ScalePtrs& sc, void* Y, void* final_state,
                                void* ws, int8_t* tap_qxs, int32_t* tap_s32, int8_t* tap_s8,
                                int8_t* tap_passed, hipStream_t st) {
  if (!fused_supported(d, dtype, int8)) return hipErrorNotSupported;
  const size_t Lp = (size_t)d.c * d.l;
  const size_t qbc = (size_t)d.B * Lp * d.G * d.N;
  const size_t cs = (size_t)d.B * d.H * d.c * d.l * sizeof(float);
  char* w = (char*)ws;
  int8_t* qB = (int8_t*)w;
  w += al(qbc);
  int8_t* qC = (int8_t*)w;
  w += al(qbc);
  int8_t* qBT = (int8_t*)w;
  w += al(qbc);
  float* dAcs = (float*)w;
  w += al(cs);
  float* lut = (float*)w;
  w += al(cs);
  uint8_t* qd = (uint8_t*)w;

  const dim3 pgrid(d.c, (unsigned)(d.B * d.G));
  if (dtype == DT_F16)
    hipLaunchKernelGGL(k_prologue_bc<DT_F16>, pgrid, dim3(256), 0, st, d, B, C, sc.inv_B, sc.inv_C, qB, qC, qBT);
  else
    hipLaunchKernelGGL(k_prologue_bc<DT_BF16>, pgrid, dim3(256), 0, st, d, B, C, sc.inv_B, sc.inv_C, qB, qC, qBT);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, qd, st);
  if (e != hipSuccess) return e;

  FusedArgs fa{d, X, dt, qB, qBT, qC, dAcs, lut, qd, D, sc, Y, (int8_t*)final_state, tap_qxs, tap_s32, tap_s8, tap_passed};
  const dim3 grid((unsigned)(d.B * d.H));
#define L_(DT_, LC_, NS_) hipLaunchKernelGGL((k_fused_i8<DT_, LC_, NS_>), grid, dim3(256), 0, st, fa)
  if (dtype == DT_F16) {
    if (d.l == 256 && d.N == 128) L_(DT_F16, 256, 128);
    else if (d.l == 256 && d.N == 64) L_(DT_F16, 256, 64);
    else if (d.l == 128 && d.N == 128) L_(DT_F16, 128, 128);
    else L_(DT_F16, 128, 64);
  } else {
    if (d.l == 256 && d.N == 128) L_(DT_BF16, 256, 128);
    else if (d.l == 256 && d.N == 64) L_(DT_BF16, 256, 64);
    else if (d.l == 128 && d.N == 128) L_(DT_BF16, 128, 128);
    else L_(DT_BF16, 128, 64);
  }
#undef L_
  return hipGetLastError();
}

}  // namespace ssd
