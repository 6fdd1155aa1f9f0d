// Fused SSD forward on the persistent-INT8 path ("SSDi8" notes page, "Overall
// framework" and "Key designs 1-3").
//
// Two prologue launches quantise B and C once per group (also writing Q(B)
// transposed per chunk) and form the float64 in-chunk cumulative sums. The main
// kernel runs one workgroup of eight waves per (batch, head). It walks that
// head's chunks in order and keeps the INT8 state in registers, so the state
// never travels through HBM. Per chunk:
//
//   Q(Xs)        X_scaled = LUT_state * x quantised once per (s, p) into LDS;
//   ChunkState   S32^T[n,p] = sum_s Q(B)^T[n,s] Q(Xs)[s,p]   (int8 MFMA; wave w
//                owns p-tile w%4 and half of the n tiles), requantised in
//                registers to S8;
//   ChunkScan1   Y_off[s,p] = sum_n Q(C)[s,n] H8_{k-1}[p,n]  (int8 MFMA, H8 in LDS);
//   ChunkBMM     CB^T tiles = Q(B) rows x Q(C) rows          (int8 MFMA; the output
//                lane layout is ChunkScan2's A-operand layout);
//   ChunkScan2   Y_diag = W x, W = CB s_C s_B exp(a_s - a_s') dt_s'  (fp16/bf16 MFMA);
//   StatePassing H8_k = sat(S8_k + RSH7(Q(Decay_k) H8_{k-1}))  (Eq. 6, in registers).
//
// The next chunk's x and Q(B) tiles are loaded into registers while the current
// chunk computes and then written to the second half of a double-buffered LDS
// area, so HBM latency overlaps the MFMA/VALU work.
//
// ChunkScan2 factorisation (exact algebra): for a column tile j strictly below
// row tile i, exp(a_s - a_s') = u_s * V_i[s'] with u_s = exp(a_s - a_{16i}) <= 1
// and V_i[s'] = exp(a_{16i} - a_s') <= 1, so each row tile needs one table V_i
// and one factor per output row instead of an exponential per element.
// Diagonal tiles use exp(a_s - a_s') directly and accumulate separately.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {
namespace {

constexpr int kP = 64;        // head dim of the fused kernel
constexpr int kThreads = 512;  // eight waves
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;

// Saturating int8 quantiser with round half away from zero. After the clamp,
// trunc(c + copysign(0.5 - 2^-25, c)) equals RHAZ(c) for every float32 c
// (checked exhaustively over all 2^32 bit patterns in the test-suite).
__device__ __forceinline__ int q8(float v) {
  const float c = fminf(fmaxf(v, -127.f), 127.f);
  return (int)(c + __builtin_copysignf(0.49999997f, c));
}

// Eq. 6 rounding shift sign(v) * ((|v| + 64) >> 7) in arithmetic-shift form:
// (v + 64 + (v >> 31)) >> 7 (equal for every |v| <= 128 * 127; tested).
__device__ __forceinline__ int rsh7_fast(int v) { return (v + 64 + (v >> 31)) >> 7; }

__device__ __forceinline__ int sat127(int v) { return min(max(v, -127), 127); }

// 2^x with the hardware transcendental (arguments here are <= 0; results that
// would be denormal flush to 0, far below anything that reaches the output).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS layouts. Rows are split into 16-byte chunks whose index is XOR-swizzled
// with low row bits, so the 8 or 16 lanes served together hit distinct banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xsw(int p) { return (p ^ (p >> 3)) & 7; }
// x transposed, [p][s] in 2-byte elements; s aligned to 4 (8-byte units). The
// two 8-byte halves of a chunk are also swapped when (p >> 3) & 1.
template <int LC>
__device__ __forceinline__ int xT_off(int p, int s) {
  return p * LC + 8 * ((s >> 3) ^ xsw(p)) + 4 * (((s >> 2) & 1) ^ ((p >> 3) & 1));
}
// byte tiles [rows][W]; c a byte column aligned to 4
template <int W>
__device__ __forceinline__ int b_off(int r, int c) {
  constexpr int nch = W / 16;
  return r * W + 16 * ((c >> 4) ^ (r & (nch - 1) & 7)) + (c & 15);
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

// ---------------------------------------------------------------------------
// Prologue: Q(B), Q(C) with padded rows (t >= L -> 0) and Q(B)^T per chunk.
// grid (c * l/64, B*G), 256 threads; one 64-row x N tile per block.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_prologue_bc(Dims d, const void* __restrict__ B,
                                                     const void* __restrict__ C,
                                                     const float* __restrict__ inv_B,
                                                     const float* __restrict__ inv_C,
                                                     int8_t* __restrict__ qB,
                                                     int8_t* __restrict__ qC,
                                                     int8_t* __restrict__ qBT) {
  constexpr int RB = 64;                 // rows per block
  constexpr int PT = RB + 4;             // LDS pitch of the transposed tile
  __shared__ __attribute__((aligned(16))) int8_t tT[128 * PT];  // [n][s]
  const int nsb = d.l / RB;
  const int k = blockIdx.x / nsb, sb = blockIdx.x % nsb;
  const int64_t bg = blockIdx.y;
  const int64_t b = bg / d.G;
  const int g = (int)(bg % d.G);
  const int N = d.N, l = d.l;
  const int64_t Lp = (int64_t)d.c * l;
  const float ib = inv_B[g], ic = inv_C[g];
  for (int item = threadIdx.x; item < RB * (N / 8); item += 256) {
    const int sl = item / (N / 8), n0 = (item % (N / 8)) * 8;
    const int64_t t = (int64_t)k * l + RB * sb + sl;
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
    for (int j = 0; j < 8; ++j) tT[(n0 + j) * PT + sl] = (int8_t)qb[j];
  }
  __syncthreads();
  // Q(B)^T rows [b][k][g][n][s]: 16 bytes per lane
  int8_t* dstT = qBT + ((b * d.c + k) * d.G + g) * (int64_t)N * l + RB * sb;
  for (int item = threadIdx.x; item < N * (RB / 16); item += 256) {
    const int n = item / (RB / 16), s0 = (item % (RB / 16)) * 16;
    const uint32_t* src = (const uint32_t*)&tT[n * PT + s0];
    *(uint4*)(dstT + (int64_t)n * l + s0) = make_uint4(src[0], src[1], src[2], src[3]);
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

template <int LC, int NS>
struct Lds {
  static constexpr int XT = kP * LC * 2;  // bytes of one x^T buffer
  static constexpr int QB = LC * NS;      // bytes of one Q(B) buffer
  static constexpr int H8 = kP * NS;
  static constexpr int VEC = 3 * LC * 4;  // a*log2(e), dt, lut (floats)
  static constexpr int VW = kWaves * LC * 4;
  static constexpr int off_xt = 0;
  static constexpr int off_qb = off_xt + 2 * XT;
  static constexpr int off_h8 = off_qb + 2 * QB;
  static constexpr int off_vec = off_h8 + H8;
  static constexpr int off_vw = off_vec + 2 * VEC;
  static constexpr int total = off_vw + VW;
};

// Registers holding the next chunk while the current one computes.
template <int LC, int NS>
struct Prefetch {
  static constexpr int XI = (LC / 4) * (kP / 8);     // x items: 4 rows x 16 bytes
  static constexpr int XPT = (XI + kThreads - 1) / kThreads;
  static constexpr int QI = LC * NS / 16;            // Q(B) 16-byte chunks
  static constexpr int QPT = QI / kThreads;
  uint4 x[XPT][4];
  uint4 q[QPT];
  float va, vd, vl;
};

template <int DT, int LC, int NS>
__device__ __forceinline__ void prefetch_load(const FusedArgs& a, int64_t b, int h, int g_h, int k,
                                              Prefetch<LC, NS>& pf) {
  typedef typename Store<DT>::T T;
  typedef Prefetch<LC, NS> PF;
  const Dims& d = a.d;
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)k * LC;
  const int64_t Lp = (int64_t)d.c * LC;
#pragma unroll
  for (int m = 0; m < PF::XPT; ++m) {
    const int item = tid + m * kThreads;
    const int q = item >> 3, c8 = item & 7;
    const int64_t tq = t0 + 4 * q;
    const T* xrow = (const T*)a.X + ((b * d.L + tq) * d.H + h) * (int64_t)kP + 8 * c8;
    const int nrow = (item < PF::XI) ? (int)min((int64_t)4, d.L - tq) : 0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      pf.x[m][r] = (r < nrow) ? *(const uint4*)(xrow + r * d.H * kP) : make_uint4(0, 0, 0, 0);
  }
  const int8_t* src = a.qB + ((b * Lp + t0) * d.G + g_h) * (int64_t)NS;
#pragma unroll
  for (int m = 0; m < PF::QPT; ++m) {
    const int id = tid + m * kThreads;
    const int s = id / (NS / 16), c16 = id % (NS / 16);
    pf.q[m] = *(const uint4*)(src + (int64_t)s * d.G * NS + 16 * c16);
  }
  if (tid < LC) {
    const int64_t ci = ((b * d.H + h) * d.c + k) * (int64_t)LC + tid;
    pf.va = a.dAcs[ci] * kLog2e;
    pf.vl = a.lut[ci];
    const int64_t t = t0 + tid;
    pf.vd = (t < d.L) ? Store<DT>::to_f(((const T*)a.dt)[(b * d.L + t) * d.H + h]) : 0.f;
  }
}

template <int LC, int NS>
__device__ __forceinline__ void prefetch_store(char* lds, int buf, const Prefetch<LC, NS>& pf) {
  typedef Lds<LC, NS> LY;
  typedef Prefetch<LC, NS> PF;
  const int tid = threadIdx.x;
  u16* xT = (u16*)(lds + LY::off_xt + buf * LY::XT);
#pragma unroll
  for (int m = 0; m < PF::XPT; ++m) {
    const int item = tid + m * kThreads;
    if (item < PF::XI) {
      const int q = item >> 3, c8 = item & 7;
      const uint32_t* w0 = (const uint32_t*)&pf.x[m][0];
      const uint32_t* w1 = (const uint32_t*)&pf.x[m][1];
      const uint32_t* w2 = (const uint32_t*)&pf.x[m][2];
      const uint32_t* w3 = (const uint32_t*)&pf.x[m][3];
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
  }
  int8_t* qb = (int8_t*)(lds + LY::off_qb + buf * LY::QB);
#pragma unroll
  for (int m = 0; m < PF::QPT; ++m) {
    const int id = tid + m * kThreads;
    const int s = id / (NS / 16), c16 = id % (NS / 16);
    *(uint4*)&qb[b_off<NS>(s, 16 * c16)] = pf.q[m];
  }
  if (tid < LC) {
    float* vec = (float*)(lds + LY::off_vec + buf * LY::VEC);
    vec[tid] = pf.va;
    vec[LC + tid] = pf.vd;
    vec[2 * LC + tid] = pf.vl;
  }
}

template <int DT, int LC, int NS>
__global__ __launch_bounds__(kThreads, 1) void k_fused_i8(FusedArgs a) {
  typedef typename Store<DT>::T T;
  typedef Lds<LC, NS> LY;
  constexpr int RT = LC / 16;      // row tiles of the chunk
  constexpr int NT = NS / 16;      // n tiles of the state
  constexpr int NTW = NT / 2;      // n tiles per wave
  constexpr int KS = LC / 64;      // ChunkState K steps
  constexpr int KN = NS / 64;      // K steps over N
  constexpr int SPT = LC / 8;      // Q(Xs) positions quantised per thread

  extern __shared__ __attribute__((aligned(16))) char lds[];
  int8_t* H8l = (int8_t*)(lds + LY::off_h8);

  const Dims& d = a.d;
  const int h = blockIdx.x % d.H;
  const int64_t b = blockIdx.x / d.H;
  const int g_h = h / d.hpg;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t Lp = (int64_t)d.c * LC;
  const int H = d.H;

  const int pt_own = w & 3;                // ChunkState / StatePassing p tile
  const int ng = w >> 2;                   // half of the n tiles
  const int p_own = 16 * pt_own + l16;
  const float mreq = a.sc.M_req[h * kP + p_own];
  const float scBC = a.sc.s_C[g_h] * a.sc.s_B[g_h];
  const float sC = a.sc.s_C[g_h];
  const float Dh = a.D[h];
  float sS[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) sS[pt] = a.sc.s_S[h * kP + 16 * pt + l16];
  // Q(Xs) quantisation role: p_q = tid % 64, positions [s_q0, s_q0 + SPT)
  const int p_q = tid & 63;
  const int s_q0 = (tid >> 6) * SPT;
  const float invx_q = a.sc.inv_X[h * kP + p_q];
  float* Vw = (float*)(lds + LY::off_vw) + w * LC;

  uint32_t H8[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) H8[j] = 0;

  {  // chunk 0 into buffer 0
    Prefetch<LC, NS> pf;
    prefetch_load<DT, LC, NS>(a, b, h, g_h, 0, pf);
    prefetch_store<LC, NS>(lds, 0, pf);
  }

  for (int k = 0; k < d.c; ++k) {
    const int cur = k & 1;
    const int64_t t0 = (int64_t)k * LC;
    const u16* xT = (const u16*)(lds + LY::off_xt + cur * LY::XT);
    const int8_t* qBl = (const int8_t*)(lds + LY::off_qb + cur * LY::QB);
    int8_t* qxs = (int8_t*)(lds + LY::off_qb + (cur ^ 1) * LY::QB);  // scratch [p][s]
    const float* vA2 = (const float*)(lds + LY::off_vec + cur * LY::VEC);
    const float* vDt = vA2 + LC;
    const float* vLut = vA2 + 2 * LC;
    __syncthreads();

    // ---- Q(X_scaled) = sat(RHAZ(fl32(fl32(lut * x) * inv_X))) into the scratch tile ----
#pragma unroll
    for (int c8 = 0; c8 < SPT / 8; ++c8) {
      const int s8 = s_q0 + 8 * c8;
      uint4 xv = *(const uint4*)&xT[xT_off<LC>(p_q, s8) & ~7];
      if ((p_q >> 3) & 1) xv = make_uint4(xv.z, xv.w, xv.x, xv.y);
      const T* xe = (const T*)&xv;
      int q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = q8((vLut[s8 + e] * Store<DT>::to_f(xe[e])) * invx_q);
      *(uint2*)&qxs[b_off<LC>(p_q, s8)] = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
      if (a.tap_qxs) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int64_t t = t0 + s8 + e;
          if (t < d.L) a.tap_qxs[((b * d.L + t) * H + h) * (int64_t)kP + p_q] = (int8_t)q[e];
        }
      }
    }
    __syncthreads();

    // ---- ChunkState^T for (p tile pt_own, n tiles ng*NTW ..) ----
    uint32_t S8[NTW];
    {
      v4i acc[NTW];
#pragma unroll
      for (int j = 0; j < NTW; ++j) acc[j] = v4i{0, 0, 0, 0};
      const int8_t* qbt = a.qBT + ((b * d.c + k) * d.G + g_h) * (int64_t)NS * LC;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int s0 = 64 * ks + 16 * lg;
        const v4i bq = *(const v4i*)&qxs[b_off<LC>(p_own, s0)];
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const int nt = ng * NTW + j;
          const v4i qa = *(const v4i*)(qbt + (int64_t)(16 * nt + l16) * LC + s0);
          acc[j] = mma_i8(qa, bq, acc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int nt = ng * NTW + j;
        if (a.tap_s32) {
          const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kP + p_own) * NS + 16 * nt + 4 * lg;
          *(int4*)(a.tap_s32 + so) = make_int4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
        }
        // requantise in registers (Key design 2)
        S8[j] = pack4(q8((float)acc[j][0] * mreq), q8((float)acc[j][1] * mreq),
                      q8((float)acc[j][2] * mreq), q8((float)acc[j][3] * mreq));
      }
    }
    __syncthreads();  // scratch free: it becomes the next chunk's Q(B) buffer

    Prefetch<LC, NS> pf;
    const bool more = k + 1 < d.c;
    if (more) prefetch_load<DT, LC, NS>(a, b, h, g_h, k + 1, pf);

    // ---- ChunkScan for row tiles {w, RT-1-w} (balanced under the causal mask) ----
#pragma unroll 1
    for (int rr = 0; rr < 2; ++rr) {
      // l = 256: tiles w and 15 - w; l = 128: tile w only
      const int i = (rr == 0) ? w : 2 * kWaves - 1 - w;
      if (i >= RT) continue;
      const int s_row = 16 * i + l16;
      v4i qc[KN];
      {
        const int8_t* src = a.qC + ((b * Lp + t0 + s_row) * d.G + g_h) * (int64_t)NS + 16 * lg;
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) qc[kn] = *(const v4i*)(src + 64 * kn);
      }
      // V_i[s'] = s_C s_B exp(a_{16i} - a_s') dt_s' for s' < 16 i (this wave's table)
      const float a_ref = vA2[16 * i];
      for (int sp = lane; sp < 16 * i; sp += kWave) Vw[sp] = scBC * fast_exp2(a_ref - vA2[sp]) * vDt[sp];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      v4f acc_off[4], acc_dg[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        acc_off[pt] = v4f{0, 0, 0, 0};
        acc_dg[pt] = v4f{0, 0, 0, 0};
      }
      // off-diagonal column tiles j < i in full pairs (jA, jA + 1); every LDS read
      // of a pair is issued before its MFMAs
#pragma unroll 2
      for (int jA = 0; jA + 1 < i; jA += 2) {
        const int jB = jA + 1;
        v4i ba[KN], bb[KN];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          ba[kn] = *(const v4i*)&qBl[b_off<NS>(16 * jA + l16, 64 * kn + 16 * lg)];
          bb[kn] = *(const v4i*)&qBl[b_off<NS>(16 * jB + l16, 64 * kn + 16 * lg)];
        }
        const float4 vA = *(const float4*)&Vw[16 * jA + 4 * lg];
        const float4 vB = *(const float4*)&Vw[16 * jB + 4 * lg];
        uint2 xa[4], xb[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          xa[pt] = *(const uint2*)&xT[xT_off<LC>(16 * pt + l16, 16 * jA + 4 * lg)];
          xb[pt] = *(const uint2*)&xT[xT_off<LC>(16 * pt + l16, 16 * jB + 4 * lg)];
        }
        v4i cbA = v4i{0, 0, 0, 0}, cbB = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          cbA = mma_i8(ba[kn], qc[kn], cbA);
          cbB = mma_i8(bb[kn], qc[kn], cbB);
        }
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
        for (int pt = 0; pt < 4; ++pt)
          acc_off[pt] = FragF<DT>::mma(af, frag_from_halves<DT>(xa[pt], xb[pt]), acc_off[pt]);
      }
      // diagonal tile j = i, sharing its MFMA with the leftover off-diagonal tile
      // j = i - 1 when i is odd (that tile's weights carry u_s so it can join the
      // unscaled diagonal accumulator: u_s V_i[s'] = exp(a_s - a_s') dt_s' s_C s_B)
      {
        const bool odd = i & 1;
        const int jL = i - 1;
        v4i bd[KN], bl[KN];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          bd[kn] = *(const v4i*)&qBl[b_off<NS>(16 * i + l16, 64 * kn + 16 * lg)];
          if (odd) bl[kn] = *(const v4i*)&qBl[b_off<NS>(16 * jL + l16, 64 * kn + 16 * lg)];
        }
        const float a_s = vA2[s_row];
        const float4 ad = *(const float4*)&vA2[16 * i + 4 * lg];
        const float4 dd = *(const float4*)&vDt[16 * i + 4 * lg];
        float4 vL = make_float4(0.f, 0.f, 0.f, 0.f);
        if (odd) vL = *(const float4*)&Vw[16 * jL + 4 * lg];
        uint2 xd[4], xl[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          xd[pt] = *(const uint2*)&xT[xT_off<LC>(16 * pt + l16, 16 * i + 4 * lg)];
          xl[pt] = odd ? *(const uint2*)&xT[xT_off<LC>(16 * pt + l16, 16 * jL + 4 * lg)] : make_uint2(0, 0);
        }
        v4i cbD = v4i{0, 0, 0, 0}, cbL = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          cbD = mma_i8(bd[kn], qc[kn], cbD);
          if (odd) cbL = mma_i8(bl[kn], qc[kn], cbL);
        }
        const float adv[4] = {ad.x, ad.y, ad.z, ad.w};
        const float ddv[4] = {dd.x, dd.y, dd.z, dd.w};
        const float us = fast_exp2(a_s - a_ref);  // u at this lane's row
        const float vLv[4] = {vL.x * us, vL.y * us, vL.z * us, vL.w * us};
        FragF<DT> af;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sp = 16 * i + 4 * lg + r;
          const float wv = (sp <= s_row) ? (float)cbD[r] * scBC * fast_exp2(a_s - adv[r]) * ddv[r] : 0.f;
          af.set(r, wv);
          af.set(r + 4, (float)cbL[r] * vLv[r]);
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          acc_dg[pt] = FragF<DT>::mma(af, frag_from_halves<DT>(xd[pt], xl[pt]), acc_dg[pt]);
      }
      // ChunkScan1 (inter-chunk)
      v4i acc1[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc1[pt] = v4i{0, 0, 0, 0};
      if (k > 0) {
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
          for (int kn = 0; kn < KN; ++kn) {
            const v4i hb = *(const v4i*)&H8l[b_off<NS>(16 * pt + l16, 64 * kn + 16 * lg)];
            acc1[pt] = mma_i8(qc[kn], hb, acc1[pt]);
          }
        }
      }
      // epilogue: rows s_out = 16 i + 4 lg + r, columns p = 16 pt + l16
      const float4 ao = *(const float4*)&vA2[16 * i + 4 * lg];
      const float aov[4] = {ao.x, ao.y, ao.z, ao.w};
      float u[4], eo[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        u[r] = fast_exp2(aov[r] - a_ref);
        eo[r] = fast_exp2(aov[r]) * sC;
      }
      const int64_t trow = t0 + 16 * i + 4 * lg;   // output row of r = 0
      T* yrow = (T*)a.Y + ((b * d.L + trow) * H + h) * (int64_t)kP + l16;
      const int ystride = H * kP;                   // elements between consecutive t
      const int nrow = (int)min((int64_t)4, d.L - trow);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const uint2 xr = *(const uint2*)&xT[xT_off<LC>(16 * pt + l16, 16 * i + 4 * lg)];
        const T* xv = (const T*)&xr;
        const float so = sS[pt];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float y = fmaf(u[r], acc_off[pt][r], acc_dg[pt][r]);
          y = fmaf(Dh, Store<DT>::to_f(xv[r]), y);
          if (k > 0) y = fmaf((float)acc1[pt][r], eo[r] * so, y);
          if (r < nrow) yrow[r * ystride + 16 * pt] = Store<DT>::from_f(y);
        }
      }
      __builtin_amdgcn_wave_barrier();  // this wave's table is rewritten by its next row tile
    }

    // next chunk into the other buffer (the scratch tile is free since the barrier above)
    if (more) prefetch_store<LC, NS>(lds, cur ^ 1, pf);
    __syncthreads();

    // ---- StatePassing (Eq. 6) in registers; publish H8 for the next ChunkScan1 ----
    {
      const int qd = a.qdecay[(b * H + h) * d.c + k];
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        const int nt = ng * NTW + j;
        if (k == 0) {
          H8[j] = S8[j];
        } else {
          int o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = sat127(byte_s(S8[j], r) + rsh7_fast(qd * byte_s(H8[j], r)));
          H8[j] = pack4(o[0], o[1], o[2], o[3]);
        }
        *(uint32_t*)&H8l[b_off<NS>(p_own, 16 * nt + 4 * lg)] = H8[j];
        const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kP + p_own) * NS + 16 * nt + 4 * lg;
        if (a.tap_s8) *(uint32_t*)(a.tap_s8 + so) = S8[j];
        if (a.tap_passed) *(uint32_t*)(a.tap_passed + so) = H8[j];
      }
    }
  }
  if (a.final_state) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int nt = ng * NTW + j;
      const int64_t fo = ((b * H + h) * (int64_t)kP + p_own) * NS + 16 * nt + 4 * lg;
      *(uint32_t*)(a.final_state + fo) = H8[j];
    }
  }
}

constexpr size_t kAl = 256;
size_t al(size_t v) { return (v + kAl - 1) / kAl * kAl; }

template <int DT, int LC, int NS>
hipError_t launch_main(const FusedArgs& fa, hipStream_t st) {
  constexpr int lds = Lds<LC, NS>::total;
  static_assert(lds <= 160 * 1024, "LDS budget");
  auto kern = k_fused_i8<DT, LC, NS>;
  static const hipError_t attr =
      hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3((unsigned)(fa.d.B * fa.d.H)), dim3(kThreads), lds, st, fa);
  return hipGetLastError();
}

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

  const dim3 pgrid((unsigned)(d.c * (d.l / 64)), (unsigned)(d.B * d.G));
  if (dtype == DT_F16)
    hipLaunchKernelGGL(k_prologue_bc<DT_F16>, pgrid, dim3(256), 0, st, d, B, C, sc.inv_B, sc.inv_C, qB, qC, qBT);
  else
    hipLaunchKernelGGL(k_prologue_bc<DT_BF16>, pgrid, dim3(256), 0, st, d, B, C, sc.inv_B, sc.inv_C, qB, qC, qBT);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, qd, st);
  if (e != hipSuccess) return e;

  const FusedArgs fa{d, X, dt, qB, qBT, qC, dAcs, lut, qd, D, sc, Y, (int8_t*)final_state,
                     tap_qxs, tap_s32, tap_s8, tap_passed};
  if (dtype == DT_F16) {
    if (d.l == 256 && d.N == 128) return launch_main<DT_F16, 256, 128>(fa, st);
    if (d.l == 256 && d.N == 64) return launch_main<DT_F16, 256, 64>(fa, st);
    if (d.l == 128 && d.N == 128) return launch_main<DT_F16, 128, 128>(fa, st);
    return launch_main<DT_F16, 128, 64>(fa, st);
  }
  if (d.l == 256 && d.N == 128) return launch_main<DT_BF16, 256, 128>(fa, st);
  if (d.l == 256 && d.N == 64) return launch_main<DT_BF16, 256, 64>(fa, st);
  if (d.l == 128 && d.N == 128) return launch_main<DT_BF16, 128, 128>(fa, st);
  return launch_main<DT_BF16, 128, 64>(fa, st);
}

}  // namespace ssd
