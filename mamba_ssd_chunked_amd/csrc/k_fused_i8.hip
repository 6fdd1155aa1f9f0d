// Fused SSD forward on the persistent-INT8 path ("SSDi8" notes page, "Overall
// framework" and "Key designs 1-3"), in two launches:
//
//  1. k_prep_cb, two kinds of blocks side by side in one launch:
//     - ChunkCumsum blocks: dAcs, LUT_state and Q(Decay) per (batch, head,
//       chunk);
//     - blocks per (batch, chunk, group), whole or in parts: Q(B) and
//       Q(C) once per group ("Key design 3"), and ChunkBMM CB = Q(C) Q(B)^T
//       on int8 MFMA (exact int32, "Key design 2": ChunkBMM reuses the int8 B
//       and C). CB depends only on (batch, chunk, group), so it is formed once
//       and shared by every head of the group. The blocks write the operands
//       of the main kernel in the register layouts its MFMAs read, so they go
//       from memory (L2) straight into registers:
//         - Q(C) rows, row-major as the inputs (ChunkScan1's operand);
//         - Q(B)^T fragments (ChunkState's operand);
//         - CB' = fp16(CB s_C s_B 2^E) fragments: ChunkScan2's weights before
//           the head's decay, with the dequantisation folded in and E a power
//           of two that keeps |CB'| < 2^15 whatever the scales
//           (|CB| <= N 127^2).
//  2. The main kernel: one 8-wave workgroup per (batch, head), or per p half
//     of a head in a last partial round, walking the head's chunks in order
//     with the int8 state in registers (it never reaches HBM). Per chunk:
//       Q(Xs)        X_scaled = LUT_state * x quantised once per (s, p) while
//                    the next chunk is staged (each wave stages an eighth of
//                    it into LDS);
//       ChunkState   S32^T[n,p] = sum_s Q(B)^T[n,s] Q(Xs)[s,p] (int8 MFMA; the
//                    Q(Xs) operand by transposing LDS reads), requantised in
//                    registers to S8;
//       ChunkScan2   Y_diag = W x, W[s,s'] = CB' exp(a_s - a_s') dt_s' 2^-E
//                    (fp16/bf16 MFMA; x by transposing LDS reads);
//       ChunkScan1   Y_off[s,p] = exp(a_s) s_C s_S[p] sum_n Q(C)[s,n] H8_{k-1}[p,n];
//       StatePassing H8_k = sat(S8_k + RSH7(Q(Decay_k) H8_{k-1})) (Eq. 6).
//
// ChunkScan2 factorisation (exact algebra): for a column tile strictly below
// row tile i, exp(a_s - a_s') = u_s V_i[s'] with u_s = exp(a_s - a_{16i}) <= 1
// and V_i[s'] = exp(a_{16i} - a_s') <= 1, so the weights of those tiles are
// CB' V_i (one mixed-precision multiply each) and u_s scales their sum once.
// The diagonal pair of column tiles uses exp(a_s - a_s') directly.
//
// Layers whose B * H heads cannot fill the GPU with one workgroup per head take
// the chunk-parallel schedule of k_chunked_i8.hip after launch 1 instead
// (ssd_shape.schedule chooses; the results are the same bit for bit).
#include "ssd_cumsum.hpp"
#include "ssd_device.hpp"
#include "ssd_fused.hpp"
#include "ssd_i8_layout.hpp"
#include "ssd_launch.hpp"

namespace ssd {
namespace {

constexpr int kCompW = 8;                     // waves per workgroup
constexpr int kCompT = kCompW * kWave;        // 512

// ===========================================================================
// Preparation launch (1024 threads per block). Blocks [0, ncs) run
// ChunkCumsum for (chunk, batch, block of kCsHeads heads). The other blocks
// write Q(C) rows, the Q(B)^T fragments of ChunkState and the CB' fragments of
// ChunkScan2, in one of three layouts:
//  - per unit (batch, chunk, group), when there are enough units to fill the
//    GPU: the chunk's Q(B) and Q(C) rows are quantised once into LDS and the
//    16 waves share the fragments;
//  - per unit half (two blocks per unit, for fewer units; cb_block_slice with
//    S = 2): each half takes the row tiles of about half the CB' fragments and
//    quantises the Q(B) rows they reach and its own Q(C) rows;
//  - per unit and pair j of row tiles {2j, 2j + 1}, for few units (more,
//    smaller blocks): Q(C) of those 32 rows and Q(B) of rows 0 .. 32 j + 31 go
//    into LDS; the block writes the Q(C) rows, the CB' fragments of the two row
//    tiles and, for odd j, the Q(B)^T fragments of K step (j - 1) / 2.
// ===========================================================================
constexpr int kPrepT = 1024;
enum { kCbPairs = 0, kCbUnit = 1, kCbHalves = 2 };  // block kinds of the B/C + ChunkBMM part
template <int LC, int NS>
struct CbLds {
  int8_t qB[LC * NS];
  int8_t qC[LC * NS];
};

template <int DT, int LC, int NS>
__device__ __forceinline__ void cb_block_unit(const Dims& d, const void* __restrict__ B, const void* __restrict__ C,
                                         const float* __restrict__ inv_B, const float* __restrict__ inv_C,
                                         const float* __restrict__ s_B, const float* __restrict__ s_C,
                                         int8_t* __restrict__ qC, int8_t* __restrict__ qbt, u16* __restrict__ cbf,
                                         int64_t unit, CbLds<LC, NS>& sm) {
  typedef typename Store<DT>::T T;
  constexpr int KN = NS / 64, NT = NS / 16, KS = LC / 64, NF = cb_frags(LC), RT = LC / 16;
  constexpr int C8 = NS / 8;                  // 8-element items per row
  constexpr int NIT = 2 * LC * C8 / kPrepT;   // items per thread (B rows, then C rows)
  static_assert(NIT * kPrepT == 2 * LC * C8, "whole items per thread");
  constexpr int NW = kPrepT / kWave;          // waves
  const int64_t g_ = unit % d.G;
  const int64_t bk = unit / d.G;
  const int k = (int)(bk % d.c);
  const int64_t b = bk / d.c;
  const int g = (int)g_;
  const int tid = threadIdx.x;
  const int64_t Lp = (int64_t)d.c * LC;
  const float ib = inv_B[g], ic = inv_C[g];

  // 1. quantise every row once: items [0, LC C8) are Q(B), the next LC C8 Q(C)
  //    (rows past L are zero; every load of a thread is issued before any is
  //    used)
  uint4 raw[NIT];
#pragma unroll
  for (int u = 0; u < NIT; ++u) {
    const int item = tid + kPrepT * u;
    const bool isB = item < LC * C8;
    const int it2 = isB ? item : item - LC * C8;
    const int s = it2 / C8, n0 = (it2 % C8) * 8;
    const int64_t t = min((int64_t)k * LC + s, d.L - 1);
    raw[u] = *(const uint4*)((const T*)(isB ? B : C) + ((b * d.L + t) * d.G + g) * (int64_t)NS + n0);
  }
#pragma unroll
  for (int u = 0; u < NIT; ++u) {
    const int item = tid + kPrepT * u;
    const bool isB = item < LC * C8;
    const int it2 = isB ? item : item - LC * C8;
    const int s = it2 / C8, n0 = (it2 % C8) * 8;
    const int64_t t = (int64_t)k * LC + s;
    const bool ok = t < d.L;
    const float inv = isB ? ib : ic;
    const uint32_t wv[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
    // sat(RHAZ(v inv)) through the clamp-then-round-away form of the main
    // kernel's quantiser (same codes as clamping after rounding; rows past L: 0)
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = ok ? Store<DT>::to_f(__builtin_bit_cast(T, (u16)(wv[e] & 0xffffu))) * inv : 0.f;
      v[2 * e + 1] = ok ? Store<DT>::to_f(__builtin_bit_cast(T, (u16)(wv[e] >> 16))) * inv : 0.f;
    }
    const uint2 pq = make_uint2(q8x4(v[0], v[1], v[2], v[3]), q8x4(v[4], v[5], v[6], v[7]));
    if (isB) {
      *(uint2*)&sm.qB[bsw<NS>(s, n0)] = pq;
    } else {
      *(uint2*)&sm.qC[bsw<NS>(s, n0)] = pq;
      *(uint2*)(qC + ((b * Lp + t) * d.G + g) * (int64_t)NS + n0) = pq;
    }
  }
  __syncthreads();
  const int w = wave_id();
  const int lane = tid & (kWave - 1);
  const int l16 = lane & 15, lg = lane >> 4;

  // 2. Q(B)^T fragments (nt, ks): lane (lg, l16) holds Q(B)[64 ks + 16 lg + e][16 nt + l16], e = 0..15
  for (int f = w; f < NT * KS; f += NW) {
    const int nt = f / KS, ks = f % KS;
    const int s0 = 64 * ks + 16 * lg, cB = 16 * nt + 8 * (l16 & 1);
    const v2i_t lo = ldtr8(sm.qB + bsw<NS>(s0 + (l16 >> 1), cB));
    const v2i_t hi = ldtr8(sm.qB + bsw<NS>(s0 + 8 + (l16 >> 1), cB));
    *(v4i*)(qbt + (unit * (NT * KS) + f) * 1024 + 16 * lane) = v4i{lo.x, lo.y, hi.x, hi.y};
  }

  // 3. CB' fragments (i, m), m = 0 .. i / 2, numbered cb_frag_base(i) + m:
  //    lane (lg, l16) holds CB'[s][s'] for s = 16 i + l16 and s' = 32 m + 16 h +
  //    4 lg + r (K slot e = 4 h + r); the two CB^T tiles (2m, 2m + 1) come out
  //    of the MFMA in exactly that layout
  const float scb = s_C[g] * s_B[g];
  const float cg = ldexpf(scb, cb_exp(scb, NS));
  for (int f = w; f < NF; f += NW) {
    int i = 0;
#pragma unroll
    for (int ii = 1; ii < RT; ++ii) i += (cb_frag_base(ii) <= f) ? 1 : 0;
    const int m = f - cb_frag_base(i);
    v4i cbA = v4i{0, 0, 0, 0}, cbB = v4i{0, 0, 0, 0};
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) {
      const v4i qcr = *(const v4i*)&sm.qC[bsw<NS>(16 * i + l16, 64 * kn + 16 * lg)];
      const v4i ba = *(const v4i*)&sm.qB[bsw<NS>(32 * m + l16, 64 * kn + 16 * lg)];
      const v4i bb = *(const v4i*)&sm.qB[bsw<NS>(32 * m + 16 + l16, 64 * kn + 16 * lg)];
      cbA = mma_i8(ba, qcr, cbA);
      cbB = mma_i8(bb, qcr, cbB);
    }
    typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
    h8_t hv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hv[r] = (_Float16)((float)cbA[r] * cg);
      hv[4 + r] = (_Float16)((float)cbB[r] * cg);
    }
    *(h8_t*)(cbf + (unit * NF + f) * 512 + 8 * lane) = hv;
  }
}

// Slices of a unit's row tiles holding about equal numbers of CB' fragments:
// slice q starts at the first row tile i with S cb_frag_base(i) >= q NF.
template <int LC, int S>
__host__ __device__ constexpr int cb_slice_tile(int q) {
  int i = 0;
  while (S * cb_frag_base(i) < q * cb_frags(LC)) ++i;
  return i;
}
// Q(B) rows the CB' fragments of row tiles below i1 reach (0 .. 32 (i1 - 1) / 2 + 31)
__host__ __device__ constexpr int cb_rows_b(int i1) { return 32 * ((i1 - 1) / 2 + 1); }

// Slice sl of S of a unit: row tiles [i0, i1). The block quantises the Q(B)
// rows its CB' fragments reach and the Q(C) rows of its tiles, writes those
// Q(C) rows and CB' fragments, and the Q(B)^T fragments of the K steps whose
// rows it covers and no earlier slice does.
template <int DT, int LC, int NS, int S>
__device__ __forceinline__ void cb_block_slice(const Dims& d, const void* __restrict__ B, const void* __restrict__ C,
                                               const float* __restrict__ inv_B, const float* __restrict__ inv_C,
                                               const float* __restrict__ s_B, const float* __restrict__ s_C,
                                               int8_t* __restrict__ qC, int8_t* __restrict__ qbt,
                                               u16* __restrict__ cbf, int64_t unit, int sl, CbLds<LC, NS>& sm) {
  typedef typename Store<DT>::T T;
  constexpr int KN = NS / 64, NT = NS / 16, KS = LC / 64, NF = cb_frags(LC), RT = LC / 16;
  constexpr int C8 = NS / 8;
  constexpr int NW = kPrepT / kWave;
  constexpr int kMaxIt = (2 * LC * C8 + kPrepT - 1) / kPrepT;
  static_assert(cb_slice_tile<LC, S>(1) > 0 && cb_slice_tile<LC, S>(S - 1) < RT, "nonempty slices");
  const int64_t g_ = unit % d.G;
  const int64_t bk = unit / d.G;
  const int k = (int)(bk % d.c);
  const int64_t b = bk / d.c;
  const int g = (int)g_;
  const int tid = threadIdx.x;
  const int64_t Lp = (int64_t)d.c * LC;
  const float ib = inv_B[g], ic = inv_C[g];
  const int i0 = cb_slice_tile<LC, S>(sl), i1 = cb_slice_tile<LC, S>(sl + 1);
  const int nB = min(LC, cb_rows_b(i1));
  const int nit = (nB + 16 * (i1 - i0)) * C8;

  // 1. quantise: items [0, nB C8) are Q(B) rows 0 .. nB - 1, the rest the Q(C)
  //    rows of tiles i0 .. i1 - 1 (rows past L are zero; every load of a thread
  //    is issued before any is used)
  uint4 raw[kMaxIt];
#pragma unroll
  for (int u = 0; u < kMaxIt; ++u) {
    const int item = tid + kPrepT * u;
    if (item < nit) {
      const bool isB = item < nB * C8;
      const int it2 = isB ? item : item - nB * C8;
      const int s = (isB ? 0 : 16 * i0) + it2 / C8, n0 = (it2 % C8) * 8;
      const int64_t t = min((int64_t)k * LC + s, d.L - 1);
      raw[u] = *(const uint4*)((const T*)(isB ? B : C) + ((b * d.L + t) * d.G + g) * (int64_t)NS + n0);
    }
  }
#pragma unroll
  for (int u = 0; u < kMaxIt; ++u) {
    const int item = tid + kPrepT * u;
    if (item < nit) {
      const bool isB = item < nB * C8;
      const int it2 = isB ? item : item - nB * C8;
      const int s = (isB ? 0 : 16 * i0) + it2 / C8, n0 = (it2 % C8) * 8;
      const int64_t t = (int64_t)k * LC + s;
      const bool ok = t < d.L;
      const float inv = isB ? ib : ic;
      const uint32_t wv[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      // sat(RHAZ(v inv)) through the clamp-then-round-away form of the main
      // kernel's quantiser (same codes as clamping after rounding; rows past L: 0)
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = ok ? Store<DT>::to_f(__builtin_bit_cast(T, (u16)(wv[e] & 0xffffu))) * inv : 0.f;
        v[2 * e + 1] = ok ? Store<DT>::to_f(__builtin_bit_cast(T, (u16)(wv[e] >> 16))) * inv : 0.f;
      }
      const uint2 pq = make_uint2(q8x4(v[0], v[1], v[2], v[3]), q8x4(v[4], v[5], v[6], v[7]));
      if (isB) {
        *(uint2*)&sm.qB[bsw<NS>(s, n0)] = pq;
      } else {
        *(uint2*)&sm.qC[bsw<NS>(s, n0)] = pq;
        *(uint2*)(qC + ((b * Lp + t) * d.G + g) * (int64_t)NS + n0) = pq;
      }
    }
  }
  __syncthreads();
  const int w = wave_id();
  const int lane = tid & (kWave - 1);
  const int l16 = lane & 15, lg = lane >> 4;

  // 2. Q(B)^T fragments (nt, ks) of K steps [ks0, ks1): those whose 64 rows this
  //    slice covers and the previous slice does not (the last slice: the rest)
  const int ks0 = sl == 0 ? 0 : min(LC, cb_rows_b(i0)) / 64;
  const int ks1 = sl == S - 1 ? KS : nB / 64;
  const int nks = ks1 - ks0;
  for (int f = w; f < NT * nks; f += NW) {
    const int nt = f / nks, ks = ks0 + f % nks;
    const int s0 = 64 * ks + 16 * lg, cB = 16 * nt + 8 * (l16 & 1);
    const v2i_t lo = ldtr8(sm.qB + bsw<NS>(s0 + (l16 >> 1), cB));
    const v2i_t hi = ldtr8(sm.qB + bsw<NS>(s0 + 8 + (l16 >> 1), cB));
    *(v4i*)(qbt + (unit * (NT * KS) + nt * KS + ks) * 1024 + 16 * lane) = v4i{lo.x, lo.y, hi.x, hi.y};
  }

  // 3. CB' fragments of row tiles i0 .. i1 - 1 (layout as in cb_block_unit)
  const float scb = s_C[g] * s_B[g];
  const float cg = ldexpf(scb, cb_exp(scb, NS));
  for (int f = cb_frag_base(i0) + w; f < cb_frag_base(i1); f += NW) {
    int i = 0;
#pragma unroll
    for (int ii = 1; ii < RT; ++ii) i += (cb_frag_base(ii) <= f) ? 1 : 0;
    const int m = f - cb_frag_base(i);
    v4i cbA = v4i{0, 0, 0, 0}, cbB = v4i{0, 0, 0, 0};
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) {
      const v4i qcr = *(const v4i*)&sm.qC[bsw<NS>(16 * i + l16, 64 * kn + 16 * lg)];
      const v4i ba = *(const v4i*)&sm.qB[bsw<NS>(32 * m + l16, 64 * kn + 16 * lg)];
      const v4i bb = *(const v4i*)&sm.qB[bsw<NS>(32 * m + 16 + l16, 64 * kn + 16 * lg)];
      cbA = mma_i8(ba, qcr, cbA);
      cbB = mma_i8(bb, qcr, cbB);
    }
    typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
    h8_t hv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hv[r] = (_Float16)((float)cbA[r] * cg);
      hv[4 + r] = (_Float16)((float)cbB[r] * cg);
    }
    *(h8_t*)(cbf + (unit * NF + f) * 512 + 8 * lane) = hv;
  }
}

template <int LC, int NS>
struct CbPairLds {
  int8_t qB[LC * NS];
  int8_t qC[32 * NS];
};

template <int DT, int LC, int NS>
__device__ __forceinline__ void cb_block_pairs(const Dims& d, const void* __restrict__ B, const void* __restrict__ C,
                                         const float* __restrict__ inv_B, const float* __restrict__ inv_C,
                                         const float* __restrict__ s_B, const float* __restrict__ s_C,
                                         int8_t* __restrict__ qC, int8_t* __restrict__ qbt, u16* __restrict__ cbf,
                                         int64_t unit, int j, CbPairLds<LC, NS>& sm) {
  typedef typename Store<DT>::T T;
  constexpr int KN = NS / 64, NT = NS / 16, KS = LC / 64, NF = cb_frags(LC);
  constexpr int C8 = NS / 8;  // 8-element items per row
  const int64_t g_ = unit % d.G;
  const int64_t bk = unit / d.G;
  const int k = (int)(bk % d.c);
  const int64_t b = bk / d.c;
  const int g = (int)g_;
  const int tid = threadIdx.x;
  const int64_t Lp = (int64_t)d.c * LC;
  const float ib = inv_B[g], ic = inv_C[g];
  const int nrB = 32 * (j + 1);  // Q(B) rows this block needs

  // 1. quantise: items [0, nrB * C8) are Q(B) rows, the next 32 * C8 the Q(C)
  //    rows 32 j .. 32 j + 31 (rows past L are zero; every load of a thread is
  //    issued before any is used)
  constexpr int kMaxIt = (LC + 32) * C8 / kPrepT + 1;
  const int nit = nrB * C8 + 32 * C8;
  uint4 raw[kMaxIt];
#pragma unroll
  for (int u = 0; u < kMaxIt; ++u) {
    const int item = tid + kPrepT * u;
    if (item < nit) {
      const bool isB = item < nrB * C8;
      const int it2 = isB ? item : item - nrB * C8;
      const int s = (isB ? 0 : 32 * j) + it2 / C8, n0 = (it2 % C8) * 8;
      const int64_t t = min((int64_t)k * LC + s, d.L - 1);
      raw[u] = *(const uint4*)((const T*)(isB ? B : C) + ((b * d.L + t) * d.G + g) * (int64_t)NS + n0);
    }
  }
#pragma unroll
  for (int u = 0; u < kMaxIt; ++u) {
    const int item = tid + kPrepT * u;
    if (item < nit) {
      const bool isB = item < nrB * C8;
      const int it2 = isB ? item : item - nrB * C8;
      const int s = (isB ? 0 : 32 * j) + it2 / C8, n0 = (it2 % C8) * 8;
      const int64_t t = (int64_t)k * LC + s;
      const bool ok = t < d.L;
      const float inv = isB ? ib : ic;
      const uint32_t wv[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      // sat(RHAZ(v inv)) through the clamp-then-round-away form of the main
      // kernel's quantiser (same codes as clamping after rounding; rows past L: 0)
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = ok ? Store<DT>::to_f(__builtin_bit_cast(T, (u16)(wv[e] & 0xffffu))) * inv : 0.f;
        v[2 * e + 1] = ok ? Store<DT>::to_f(__builtin_bit_cast(T, (u16)(wv[e] >> 16))) * inv : 0.f;
      }
      const uint2 pq = make_uint2(q8x4(v[0], v[1], v[2], v[3]), q8x4(v[4], v[5], v[6], v[7]));
      if (isB) {
        *(uint2*)&sm.qB[bsw<NS>(s, n0)] = pq;
      } else {
        *(uint2*)&sm.qC[bsw<NS>(s - 32 * j, n0)] = pq;
        *(uint2*)(qC + ((b * Lp + t) * d.G + g) * (int64_t)NS + n0) = pq;
      }
    }
  }
  __syncthreads();
  const int w = wave_id();
  const int lane = tid & (kWave - 1);
  const int l16 = lane & 15, lg = lane >> 4;

  // 2. Q(B)^T fragments of K step ks = (j - 1) / 2 (odd j): fragment (nt, ks),
  //    lane (lg, l16) holds Q(B)[64 ks + 16 lg + e][16 nt + l16], e = 0..15
  if ((j & 1) && w < NT) {
    const int nt = w, ks = (j - 1) / 2;
    const int s0 = 64 * ks + 16 * lg, cB = 16 * nt + 8 * (l16 & 1);
    const v2i_t lo = ldtr8(sm.qB + bsw<NS>(s0 + (l16 >> 1), cB));
    const v2i_t hi = ldtr8(sm.qB + bsw<NS>(s0 + 8 + (l16 >> 1), cB));
    *(v4i*)(qbt + (unit * (NT * KS) + nt * KS + ks) * 1024 + 16 * lane) = v4i{lo.x, lo.y, hi.x, hi.y};
  }

  // 3. CB' fragments (i, m) of row tiles i = 2j, 2j + 1, m = 0 .. j (one per
  //    wave): lane (lg, l16) holds CB'[s][s'] for s = 16 i + l16 and s' =
  //    32 m + 16 h + 4 lg + r (K slot e = 4 h + r); the two CB^T tiles
  //    (2m, 2m + 1) come out of the MFMA in exactly that layout
  if (w < 2 * (j + 1)) {
    const int i = 2 * j + w / (j + 1), m = w % (j + 1);
    const float scb = s_C[g] * s_B[g];
    const float cg = ldexpf(scb, cb_exp(scb, NS));
    v4i cbA = v4i{0, 0, 0, 0}, cbB = v4i{0, 0, 0, 0};
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) {
      const v4i qcr = *(const v4i*)&sm.qC[bsw<NS>(16 * (i - 2 * j) + l16, 64 * kn + 16 * lg)];
      const v4i ba = *(const v4i*)&sm.qB[bsw<NS>(32 * m + l16, 64 * kn + 16 * lg)];
      const v4i bb = *(const v4i*)&sm.qB[bsw<NS>(32 * m + 16 + l16, 64 * kn + 16 * lg)];
      cbA = mma_i8(ba, qcr, cbA);
      cbB = mma_i8(bb, qcr, cbB);
    }
    typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
    h8_t hv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hv[r] = (_Float16)((float)cbA[r] * cg);
      hv[4 + r] = (_Float16)((float)cbB[r] * cg);
    }
    *(h8_t*)(cbf + (unit * NF + cb_frag_base(i) + m) * 512 + 8 * lane) = hv;
  }
}

template <int LC, int NS>
struct PrepLds {
  static constexpr size_t kCb = sizeof(CbLds<LC, NS>) > sizeof(CbPairLds<LC, NS>) ? sizeof(CbLds<LC, NS>)
                                                                                     : sizeof(CbPairLds<LC, NS>);
  static constexpr size_t kBytes = sizeof(CsLds) > kCb ? sizeof(CsLds) : kCb;
};

template <int DT, int LC, int NS>
__global__ __launch_bounds__(kPrepT) void k_prep_cb(Dims d, const void* __restrict__ dt, const float* __restrict__ A,
                                                    float* __restrict__ dAcs, float* __restrict__ lut,
                                                    uint8_t* __restrict__ qdecay, const void* __restrict__ B,
                                                    const void* __restrict__ C, const float* __restrict__ inv_B,
                                                    const float* __restrict__ inv_C, const float* __restrict__ s_B,
                                                    const float* __restrict__ s_C, int8_t* __restrict__ qC,
                                                    int8_t* __restrict__ qbt, u16* __restrict__ cbf, int ncs,
                                                    int cb_kind) {
  static_assert(kPrepT == kCsThreads, "one block size for both kinds");
  __shared__ __attribute__((aligned(16))) char lds[PrepLds<LC, NS>::kBytes];
  const int64_t bi = blockIdx.x;
  if (bi < ncs) {
    const int k = (int)(bi % d.c);
    const int64_t rest = bi / d.c;
    chunk_cumsum_block<DT>(dt, A, dAcs, lut, qdecay, d, k, rest % d.B, (int)(rest / d.B), *(CsLds*)lds);
  } else {
    const int64_t ci = bi - ncs;
    // the B/C + ChunkBMM blocks are the launch's long pole; where they share a
    // CU with cumsum blocks they issue first (measured: 16.0 -> 15.0 us on the
    // 2.7B layer, 40.0 -> 38.5 and 41.2 -> 38.9 on the 8B and 64K-token ones)
    __builtin_amdgcn_s_setprio(1);
    constexpr int NJ = LC / 32;
    if (cb_kind == kCbUnit)
      cb_block_unit<DT, LC, NS>(d, B, C, inv_B, inv_C, s_B, s_C, qC, qbt, cbf, ci, *(CbLds<LC, NS>*)lds);
    else if (cb_kind == kCbHalves)
      cb_block_slice<DT, LC, NS, 2>(d, B, C, inv_B, inv_C, s_B, s_C, qC, qbt, cbf, ci >> 1, (int)(ci & 1),
                                    *(CbLds<LC, NS>*)lds);

    else
      cb_block_pairs<DT, LC, NS>(d, B, C, inv_B, inv_C, s_B, s_C, qC, qbt, cbf, ci / NJ, (int)(ci % NJ),
                                 *(CbPairLds<LC, NS>*)lds);
  }
}

// ===========================================================================
// main kernel
// ===========================================================================
struct I8Args {
  Dims d;
  const void* X;
  const void* dt;
  const int8_t* qC;
  const int8_t* qbt;
  const u16* cbf;
  const float* dAcs;
  const float* lut;
  const uint8_t* qdecay;
  const float* D;
  ScalePtrs sc;
  void* Y;
  const int8_t* init;  // optional initial state [B,H,P,N] (the passed state before chunk 0)
  int8_t* final_state;
  int8_t* tap_qxs;
  int32_t* tap_s32;
  int8_t* tap_s8;
  int8_t* tap_passed;
  int64_t nfull;
  int unit_map;
  int half_il;
};

// Staging registers of one wave for one chunk: its share of the chunk is rows
// s = (l / 8) w + lane / R + (64 / R) u (u = 0 .. NU - 1) of the block's p
// range, each lane 8 columns of a row (R = 8 lanes per row for a whole head,
// 4 for a p half), with LUT_state of those rows, and for lanes below l / 8
// the dAcs and dt of position (l / 8) w + lane.
template <int NU_>
struct SRegs {
  static constexpr int NU = NU_;
  v4i x[NU];
  float lut[NU];
  float va;
  uint32_t vd;
  uint32_t qd;  // the dword holding the chunk's Q(Decay) byte
};

// A row tile's operands as its scan reads them: the m-th off-diagonal CB'
// fragment (m below MF) is F[m], or F[NF_ - 1 - m] for the second row tile of a
// wave, whose fragments fill the register array from the top.
template <int MF_, int NF_, bool REV, int KN>
struct TileView {
  static constexpr int MF = MF_;
  const v4i (&F)[NF_];
  const v4i& diag;
  const v4i (&qc)[KN];
  __device__ __forceinline__ const v4i& off(int m) const { return REV ? F[NF_ - 1 - m] : F[m]; }
};

template <int DT, int LC, int NS, int PW, bool TAPS>
__device__ __forceinline__ void fused_i8_v2(const I8Args& a, const int64_t bx, u16* s_x, int8_t* s_qx,
                                            int8_t* s_h8, float* s_va, float* s_vb, float* s_vw,
                                            float* s_ss, int* s_qd) {
  typedef typename Store<DT>::T T;
  typedef FragF<DT> F;
  constexpr int RT = LC / 16;              // row tiles of the chunk
  constexpr int NT = NS / 16;              // n tiles of the state
  constexpr int PTW = PW * NT / kCompW;    // p tiles per wave in ChunkState / StatePassing
  constexpr int KS = LC / 64;              // ChunkState K steps
  constexpr int KN = NS / 64;              // K steps over N
  constexpr int NF = cb_frags(LC);
  constexpr int XN = LC * kHP, QN = LC * kHP, HN = kHP * NS;
  constexpr int NRR = (LC == 256) ? 2 : 1;  // row tiles per wave
  constexpr int SR = LC / 8;                // staged rows per wave
  constexpr int LPR = 2 * PW;               // staging lanes per row (the block's p range, 16 bytes each)
  constexpr int RPP = kWave / LPR;          // rows per staging pass
  constexpr int NU = SR / RPP;              // staging passes per chunk
  static_assert(NU * RPP == SR, "whole staging passes");
  const Dims& d = a.d;
  const BlockHead bh = block_head<PW>(d, bx, a.nfull, a.unit_map, a.half_il);
  const int pt_base = (PW == 4) ? 0 : 2 * bh.ph;
  const int64_t b = bh.unit / d.G;
  const int g_h = (int)(bh.unit % d.G);
  const int h = g_h * d.hpg + (int)bh.hl;
  const int H = d.H;
  const int64_t Lp = (int64_t)d.c * LC;
  const int w = wave_id();
  const int tid0 = threadIdx.x;
  const int lane = tid0 & (kWave - 1);
  const int l16 = lane & 15, lg = lane >> 4;
  const bool has_init = a.init != nullptr;
  const float scb = a.sc.s_C[g_h] * a.sc.s_B[g_h];
  const float Eg = (float)cb_exp(scb, NS);
  const int nt_own = w % NT;
  const int pt0 = pt_base + (w / NT) * PTW;
  const float sC = a.sc.s_C[g_h];
  const float Dh = a.D[h];
  const int64_t bh_ = b * H + h;
  T* const ybase = (T*)a.Y + (b * d.L * H + h) * (int64_t)kHP;
  float* Vw = s_vw + w * LC;

  if (tid0 < kHP) {
    s_ss[tid0] = a.sc.s_S[h * kHP + tid0];
    s_ss[2 * kHP + tid0] = a.sc.M_req[h * kHP + tid0];
  }

  // ---- staging of a chunk (each wave its share) ----
  // a p half stages only its own columns: its ChunkState and ChunkScan read no others
  const int c8 = 2 * pt_base + (lane & (LPR - 1)), sr0 = SR * w + lane / LPR;
  const int sv = SR * w + (lane & (SR - 1));  // this lane's position for the per-position values
  const int64_t rowB = (int64_t)H * kHP * sizeof(T);
  const char* xh = (const char*)a.X + (b * d.L * H + h) * (int64_t)kHP * sizeof(T);
  const uint32_t x_lane = (uint32_t)(16 * c8);
  // (real == false: the same loads from the chunk's first row, L2-resident
  // and never used, so that every chunk issues the same vector-memory
  // operations and the compiler's in-order wait counts stay exact)
  const auto stage_load = [&](int kc, SRegs<NU>& r, bool real) {
    const int64_t t0 = (int64_t)kc * LC;
    const int64_t cs0 = (bh_ * d.c + kc) * (int64_t)LC;
    const int64_t lim = real ? d.L - 1 - t0 : 0;  // last valid row of the chunk
    const int srow = real ? sr0 : 0, svr = real ? sv : 0;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int64_t s = min((int64_t)(srow + (real ? RPP * u : 0)), lim);
      r.x[u] = __builtin_nontemporal_load((const v4i*)(xh + (t0 + s) * rowB + x_lane));
      r.lut[u] = a.lut[cs0 + s];
    }
    r.va = a.dAcs[cs0 + svr];
    const int64_t tv = t0 + min((int64_t)svr, lim);
    if constexpr (sizeof(T) == 4)
      r.vd = *(const uint32_t*)((const T*)a.dt + (b * d.L + tv) * H + h);
    else
      r.vd = *(const u16*)((const T*)a.dt + (b * d.L + tv) * H + h);
    r.qd = *(const uint32_t*)(a.qdecay + ((bh_ * d.c + kc) & ~(int64_t)3));
  };
  const float4 ix0 = ld_scale4(&a.sc.inv_X[h * kHP + 8 * c8]);
  const float4 ix1 = ld_scale4(&a.sc.inv_X[h * kHP + 8 * c8 + 4]);
  const float ix[8] = {ix0.x, ix0.y, ix0.z, ix0.w, ix1.x, ix1.y, ix1.z, ix1.w};
  const auto stage_store = [&](int kc, const SRegs<NU>& r) {
    const int o = kc & 1;
    u16* xw = s_x + o * XN;
    int8_t* qw = s_qx + o * QN;
    const int64_t t0 = (int64_t)kc * LC;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int s = sr0 + RPP * u;
      *(v4i*)&xw[xsw_off(s, 8 * c8)] = r.x[u];
      // Q(X_scaled) = sat(RHAZ(fl32(fl32(lut * x) * inv_X))) ("Key design 1");
      // rows past L have LUT_state 0, so their codes are 0
      const uint32_t wv[4] = {(uint32_t)r.x[u][0], (uint32_t)r.x[u][1], (uint32_t)r.x[u][2], (uint32_t)r.x[u][3]};
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = Store<DT>::to_f(__builtin_bit_cast(T, (u16)(wv[j] & 0xffffu)));
        const float x1 = Store<DT>::to_f(__builtin_bit_cast(T, (u16)(wv[j] >> 16)));
        v[2 * j] = __builtin_fmaf(r.lut[u], x0, 0.0f) * ix[2 * j];
        v[2 * j + 1] = __builtin_fmaf(r.lut[u], x1, 0.0f) * ix[2 * j + 1];
      }
      const uint2 q = make_uint2(q8x4(v[0], v[1], v[2], v[3]), q8x4(v[4], v[5], v[6], v[7]));
      *(uint2*)&qw[qsw_off(s, 8 * c8)] = q;
      if (TAPS && a.tap_qxs && t0 + s < d.L)
        *(uint2*)(a.tap_qxs + ((b * d.L + t0 + s) * H + h) * (int64_t)kHP + 8 * c8) = q;
    }
    if (lane < SR) {
      float dtv;
      if constexpr (sizeof(T) == 4)
        dtv = __uint_as_float(r.vd);
      else
        dtv = Store<DT>::to_f(__builtin_bit_cast(T, (u16)r.vd));
      if (t0 + sv >= d.L) dtv = 0.f;
      float A2, B2;
      scan_vectors(r.va, dtv, Eg, A2, B2);
      s_va[o * LC + sv] = A2;
      s_vb[o * LC + kperm(sv)] = B2;
    }
    // Q(Decay) of the chunk, for its StatePassing (through LDS, so no value
    // loaded in one chunk is carried in a register into the next)
    if (w == 0 && lane == 0) s_qd[o] = (int)((r.qd >> (8 * ((bh_ * d.c + kc) & 3))) & 0xff);
  };

  // per-lane LDS offsets of the transposing reads (see xsw_off / qsw_off)
  int xoff[PW];  // ChunkScan2 x operand of p tile pt_base + jp, rows 4 lg + (l16 >> 2) (+ 32 m + 16 h)
#pragma unroll
  for (int jp = 0; jp < PW; ++jp) xoff[jp] = xsw_off(4 * lg + (l16 >> 2), 16 * (pt_base + jp) + 4 * (l16 & 3));
  int qoff[PTW];  // ChunkState Q(Xs) operand of p tile pt0 + j, rows 16 lg + (l16 >> 1) (+ 64 ks + 8 h)
#pragma unroll
  for (int j = 0; j < PTW; ++j) qoff[j] = qsw_off(16 * lg + (l16 >> 1), 16 * (pt0 + j) + 8 * (l16 & 1));

  uint32_t H8[PTW];  // passed state: lane (p = 16 (pt0 + j) + l16, n = 16 nt_own + 4 lg + r)
#pragma unroll
  for (int j = 0; j < PTW; ++j) {
    const int p = 16 * (pt0 + j) + l16;
    H8[j] = has_init ? *(const uint32_t*)(a.init + (bh_ * kHP + p) * NS + 16 * nt_own + 4 * lg) : 0u;
    // the initial state feeds chunk 0's ChunkScan1 (buffer (0 - 1) & 1)
    if (has_init) *(uint32_t*)&s_h8[HN + bsw<NS>(p, 16 * nt_own + 4 * lg)] = H8[j];
  }

  // Global operands: a wave-uniform base plus a 32-bit lane offset.
  const uint32_t lane16 = 16u * (uint32_t)lane;  // fragment byte offset of this lane
  const char* const qbt_h = (const char*)a.qbt + ((int64_t)(b * d.c * d.G + g_h) * (NT * KS) + nt_own * KS) * 1024;
  const int64_t qbt_kstride = (int64_t)d.G * (NT * KS) * 1024;  // per chunk
  const char* const cbf_h = (const char*)a.cbf + (int64_t)(b * d.c * d.G + g_h) * NF * 1024;
  const int64_t cbf_kstride = (int64_t)d.G * NF * 1024;
  const auto frag = [&](const char* base) { return *(const v4i*)(base + lane16); };
  const auto load_qbt = [&](int kc, v4i (&q)[KS]) {
    const char* src = qbt_h + kc * qbt_kstride;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) q[ks] = frag(src + ks * 1024);
  };
  const uint32_t qc_lane = (uint32_t)(l16 * d.G * NS + 16 * lg);
  const auto load_qc = [&](int kc, int i, v4i (&q)[KN]) {
    const int8_t* src = a.qC + ((b * Lp + (int64_t)kc * LC + 16 * i) * d.G + g_h) * (int64_t)NS;
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) q[kn] = *(const v4i*)(src + (qc_lane + 64 * kn));
  };
  // A row tile's operands from memory: its CB' fragments (off-diagonal pairs
  // and the diagonal one) and Q(C) rows, issued one phase ahead of their use and
  // always before this wave's Y stores of the phase in between (the vector
  // memory counter retires in issue order, so a wait for an operand then never
  // waits for a store). Every wave issues the same number of loads at the same
  // points, so the compiler's in-order wait counts stay exact.
  //  - One row tile per wave (l = 128): tile w has w / 2 <= 3 off-diagonal
  //    pairs; the slots past them reload the diagonal fragment (cached).
  //  - Two row tiles per wave (l = 256): tiles w and 15 - w have w / 2 and
  //    7 - w / 2 pairs, 7 together, held in Fo[0 .. 6]: the first tile's
  //    fragments from the bottom, the second's from the top. Fo[0 .. 3] (the
  //    first tile's pairs and the second's highest ones) and the first tile's
  //    diagonal and Q(C) come at the barrier; Fo[4 .. 6] and the second tile's
  //    diagonal and Q(C) after the first tile.
  constexpr int NOFF = (NRR == 2) ? RT / 2 - 1 : 4;
  static_assert(NRR == 1 || RT == 2 * kCompW, "two row tiles per wave pair up as w and RT - 1 - w");
  const auto frag_src = [&](int kc, int i) { return cbf_h + kc * cbf_kstride + cb_frag_base(i) * 1024; };
  const auto load_first = [&](int kc, int i1, v4i (&Fo)[NOFF], v4i& diag, v4i (&qc)[KN]) {
    const int mi1 = i1 >> 1;
    const char* s1 = frag_src(kc, i1);
    if constexpr (NRR == 2) {
      const char* s2 = frag_src(kc, RT - 1 - i1);
#pragma unroll
      for (int j = 0; j < 4; ++j) Fo[j] = frag(j < mi1 ? s1 + j * 1024 : s2 + (NOFF - 1 - j) * 1024);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) Fo[j] = frag(s1 + min(j, mi1) * 1024);
    }
    diag = frag(s1 + mi1 * 1024);
    load_qc(kc, i1, qc);
  };
  const auto load_second = [&](int kc, int i2, v4i (&Fo)[NOFF], v4i& diag, v4i (&qc)[KN]) {
    const char* s2 = frag_src(kc, i2);
#pragma unroll
    for (int j = NOFF - 1; j >= 4; --j) Fo[j] = frag(s2 + (NOFF - 1 - j) * 1024);
    diag = frag(s2 + (i2 >> 1) * 1024);
    load_qc(kc, i2, qc);
  };

  // prologue: stage chunk 0 (every wave its share)
  {
    SRegs<NU> r;
    stage_load(0, r, true);
    stage_store(0, r);
  }
  v4i qbt[KS];
  load_qbt(0, qbt);

  for (int k = 0; k < d.c; ++k) {
    const int o = k & 1;
    const u16* xb = s_x + o * XN;
    const int8_t* qxb = s_qx + o * QN;
    const float* vA = s_va + o * LC;
    const float* vB = s_vb + o * LC;
    const int8_t* h8r = s_h8 + (o ^ 1) * HN;  // H_{k-1}
    int8_t* h8w = s_h8 + o * HN;              // H_k
    const int kn1 = min(k + 1, d.c - 1);      // next chunk (clamped; the last chunk prefetches nothing)
    const int64_t t0 = (int64_t)k * LC;
    __syncthreads();  // B1: chunk k staged; H_{k-1} published; chunk k - 1's buffers free
    // the wave index, hidden from the compiler at every chunk: values derived
    // from it (row tiles, fragment offsets, which pairs are below the
    // diagonal) are then formed per chunk in scalar registers instead of being
    // hoisted out of the loop and spilled
    int wk = w;
    asm volatile("" : "+s"(wk));
    // Issue priority: waves w and w + 4 share a SIMD, and the arbiter favours
    // the older one, so the second fell behind by about 2,000 cycles per chunk
    // and ran alone at the end while the first waited at the barrier. The
    // second wave now leads the first half of the chunk (ChunkState and the
    // first row tile) and the first wave the second half (measured: 3-5%
    // faster on the 2.7B layer; leading the second wave for the whole chunk,
    // switching after ChunkState, alternating by chunk or switching four
    // times per chunk gained less).
    if (wk >= 4) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
    // the first row tile's operands (landing during ChunkState) and the next
    // chunk's share of x (landing by the time it is staged); the second row
    // tile's operands are issued after the first tile, so that the burst at
    // the barrier stays short
    v4i Fo[NOFF], diag1, diag2, qc1[KN], qc2[KN];
    load_first(k, wk, Fo, diag1, qc1);
    SRegs<NU> sreg;
    stage_load(kn1, sreg, k + 1 < d.c);

    v2s S8a[PTW], S8b[PTW];
    // ---- ChunkState^T for (n tile nt_own, p tiles pt0 ..), requantised to S8 ----
    // (the Q(Xs) operands of step ks + 1 are read while step ks multiplies)
    const auto chunk_state = [&]() {
      v4i acc[PTW];
      v4i bq[2][PTW];
      const auto rd = [&](int ks, v4i(&dst)[PTW]) {
#pragma unroll
        for (int j = 0; j < PTW; ++j) {
          const v2i_t lo = ldtr8(qxb + qoff[j] + (64 * ks) * kHP);
          const v2i_t hi = ldtr8(qxb + qoff[j] + (64 * ks + 8) * kHP);
          dst[j] = v4i{lo.x, lo.y, hi.x, hi.y};
        }
      };
      rd(0, bq[0]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) rd(ks + 1, bq[(ks + 1) & 1]);
#pragma unroll
        for (int j = 0; j < PTW; ++j)
          acc[j] = mma_i8(qbt[ks], bq[ks & 1][j], ks == 0 ? v4i{0, 0, 0, 0} : acc[j]);
      }
#pragma unroll
      for (int j = 0; j < PTW; ++j) {
        const int p = 16 * (pt0 + j) + l16;
        if (TAPS && a.tap_s32) {
          const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kHP + p) * NS + 16 * nt_own + 4 * lg;
          *(int4*)(a.tap_s32 + so) = make_int4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
        }
        // requantise in registers ("Key design 2"); codes kept as int16 pairs
        const float mreq = s_ss[2 * kHP + p];
        S8a[j] = cvt_pair(q8_pre((float)acc[j][0] * mreq), q8_pre((float)acc[j][1] * mreq));
        S8b[j] = cvt_pair(q8_pre((float)acc[j][2] * mreq), q8_pre((float)acc[j][3] * mreq));
      }
    };

    // ---- ChunkScan, transposed: Y^T[p, s] for row tile i ----
    const auto scan_tile = [&](const int i, const auto& t, auto after_offdiag) {
      constexpr int MF = std::remove_reference_t<decltype(t)>::MF;
      const int mi = i >> 1;  // pairs 0 .. mi - 1 are below the diagonal; pair mi holds it
      const int s_row = 16 * i + l16;
      const float a_ref = vA[16 * i];
      // V_i[s'] dt_s' 2^-E for s' < 32 mi, stored by K slot (kperm): exp2(a_ref - B)
      for (int qq = lane; qq < 32 * mi; qq += kWave) Vw[qq] = __builtin_amdgcn_exp2f(a_ref - vB[qq]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      v4f acc[PW];
#pragma unroll
      for (int jp = 0; jp < PW; ++jp) acc[jp] = v4f{0, 0, 0, 0};
      const auto xfrags = [&](int m, F(&xf)[PW]) {
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) {
          const v4s_t lo = ldtr16(xb + xoff[jp] + (32 * m) * kHP);
          const v4s_t hi = ldtr16(xb + xoff[jp] + (32 * m + 16) * kHP);
          xf[jp].v = __builtin_bit_cast(decltype(xf[jp].v), v8s_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
      };
      // off-diagonal pairs: W = CB' V (one mixed-precision multiply per weight);
      // the x operands are read first, so their latency overlaps the weights
#pragma unroll
      for (int m = 0; m < MF; ++m) {
        if (m < mi) {
          F xf[PW];
          xfrags(m, xf);
          const float4 va = *(const float4*)&Vw[32 * m + 8 * lg];
          const float4 vb = *(const float4*)&Vw[32 * m + 8 * lg + 4];
          const float vv[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
          const v4i cw = t.off(m);
          F wf;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t dw = (uint32_t)cw[e >> 1];
            const _Float16 c16 = __builtin_bit_cast(_Float16, (u16)((e & 1) ? (dw >> 16) : (dw & 0xffffu)));
            wf.set(e, __builtin_fmaf((float)c16, vv[e], 0.0f));
          }
#pragma unroll
          for (int jp = 0; jp < PW; ++jp) acc[jp] = F::mma(xf[jp], wf, acc[jp]);
        }
      }
      after_offdiag();
      const float a_s = vA[s_row];
      const float us = __builtin_amdgcn_exp2f(a_s - a_ref);
#pragma unroll
      for (int jp = 0; jp < PW; ++jp) acc[jp] *= us;
      // ChunkScan1 (inter-chunk): H8 rows x Q(C) rows, scaled by exp(a_s) s_C s_S[p]
      if (k > 0 || has_init) {
        const float eo = __builtin_amdgcn_exp2f(a_s) * sC;
        v4i acc1[PW];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          v4i hb[PW];
#pragma unroll
          for (int jp = 0; jp < PW; ++jp)
            hb[jp] = *(const v4i*)&h8r[bsw<NS>(16 * (pt_base + jp) + l16, 64 * kn + 16 * lg)];
#pragma unroll
          for (int jp = 0; jp < PW; ++jp) acc1[jp] = mma_i8(hb[jp], t.qc[kn], kn == 0 ? v4i{0, 0, 0, 0} : acc1[jp]);
        }
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) {
          const float4 ss = *(const float4*)&s_ss[16 * (pt_base + jp) + 4 * lg];
          acc[jp][0] = fmaf((float)acc1[jp][0], eo * ss.x, acc[jp][0]);
          acc[jp][1] = fmaf((float)acc1[jp][1], eo * ss.y, acc[jp][1]);
          acc[jp][2] = fmaf((float)acc1[jp][2], eo * ss.z, acc[jp][2]);
          acc[jp][3] = fmaf((float)acc1[jp][3], eo * ss.w, acc[jp][3]);
        }
      }
      // diagonal pair mi: exp(a_s - a_s') dt_s' 2^-E directly (zero above the
      // diagonal), with D on the diagonal so the skip term D x rides the MFMA
      // An even tile (i = 2 mi) has its diagonal block in the pair's first
      // column tile and only zero weights in the second (above the
      // diagonal), so that half takes no exps and no x reads: its weights
      // and x slots are written as zeros, which leaves every product, and
      // so Y, bit for bit as with the full pair.
      {
        const bool even = (i & 1) == 0;
        const float4 ba = *(const float4*)&vB[32 * mi + 8 * lg];
        const float bva[4] = {ba.x, ba.y, ba.z, ba.w};
        F wf;
        const auto diag_w = [&](int e, float bvv) {
          const int sp = 32 * mi + 16 * (e >> 2) + 4 * lg + (e & 3);
          const float arg = (sp <= s_row) ? a_s - bvv : -__builtin_inff();
          const float ev = __builtin_amdgcn_exp2f(arg);
          const uint32_t dw = (uint32_t)t.diag[e >> 1];
          const _Float16 c16 = __builtin_bit_cast(_Float16, (u16)((e & 1) ? (dw >> 16) : (dw & 0xffffu)));
          wf.set(e, __builtin_fmaf((float)c16, ev, (sp == s_row) ? Dh : 0.0f));
        };
#pragma unroll
        for (int e = 0; e < 4; ++e) diag_w(e, bva[e]);
        if (even) {
#pragma unroll
          for (int e = 4; e < 8; ++e) wf.set(e, 0.0f);
        } else {
          const float4 bb = *(const float4*)&vB[32 * mi + 8 * lg + 4];
          const float bvb[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
          for (int e = 4; e < 8; ++e) diag_w(e, bvb[e - 4]);
        }
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) {
          const v4s_t lo = ldtr16(xb + xoff[jp] + (32 * mi) * kHP);
          v4s_t hi = v4s_t{0, 0, 0, 0};
          if (!even) hi = ldtr16(xb + xoff[jp] + (32 * mi + 16) * kHP);
          F xd;
          xd.v = __builtin_bit_cast(decltype(xd.v), v8s_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          acc[jp] = F::mma(xd, wf, acc[jp]);
        }
      }
      // epilogue: lane holds s = s_row and p = 16 pt + 4 lg + r
      {
        // lanes of rows lg and lg ^ 1 (same l16) swap halves so that each lane
        // holds whole 16-byte pieces (8 consecutive p) and stores half as often
        uint32_t dv[PW][2];
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) {
          dv[jp][0] = pack2<DT>(acc[jp][0], acc[jp][1]);
          dv[jp][1] = pack2<DT>(acc[jp][2], acc[jp][3]);
        }
        const bool odd = lg & 1;
        const uint32_t om = odd ? 0xffffffffu : 0u;  // bitwise selects (no indexed register arrays)
        constexpr int HP = PW / 2;  // p tiles a lane sends (and keeps)
        uint32_t rv[HP][2], kv[HP][2];
#pragma unroll
        for (int q = 0; q < HP; ++q)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const uint32_t v = (dv[q][e] & om) | (dv[HP + q][e] & ~om);  // odd rows send p tile q, even ones HP + q
            kv[q][e] = (dv[HP + q][e] & om) | (dv[q][e] & ~om);          // and keep the other
            const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
            rv[q][e] = (r[0] & om) | (r[1] & ~om);
          }
        if (t0 + s_row < d.L) {
          char* yrow = (char*)(ybase + (t0 + s_row) * (int64_t)H * kHP) + 32 * pt_base + 8 * (lg & 2);
#pragma unroll
          for (int q = 0; q < HP; ++q) {
            const int jp = odd ? HP + q : q;
            // the lower 8 bytes come from the even row, the upper from the odd one
            const uint32_t l0 = (rv[q][0] & om) | (kv[q][0] & ~om), l1 = (rv[q][1] & om) | (kv[q][1] & ~om);
            const uint32_t h0 = (kv[q][0] & om) | (rv[q][0] & ~om), h1 = (kv[q][1] & om) | (rv[q][1] & ~om);
            const v4i piece = v4i{(int)l0, (int)l1, (int)h0, (int)h1};
            *(v4i*)(yrow + 32 * jp) = piece;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();  // this wave's table is rewritten by its next row tile
    };

    chunk_state();
    // the next chunk's Q(B)^T fragments are issued after the last tile's
    // off-diagonal pairs, ahead of its Y stores; the next chunk's share is
    // staged into the other buffer (its readers, chunk k - 1, are past B1)
    const auto next_qbt = [&] { load_qbt(kn1, qbt); };  // the last chunk reloads its own (L2-resident)
    if constexpr (NRR == 2) {
      scan_tile(wk, TileView<4, NOFF, false, KN>{Fo, diag1, qc1}, [] {});
      load_second(k, RT - 1 - wk, Fo, diag2, qc2);
      if (wk >= 4) __builtin_amdgcn_s_setprio(0); else __builtin_amdgcn_s_setprio(1);
      if (k + 1 < d.c) stage_store(k + 1, sreg);
      scan_tile(RT - 1 - wk, TileView<NOFF, NOFF, true, KN>{Fo, diag2, qc2}, next_qbt);
    } else {
      scan_tile(wk, TileView<4, NOFF, false, KN>{Fo, diag1, qc1}, next_qbt);
      if (wk >= 4) __builtin_amdgcn_s_setprio(0); else __builtin_amdgcn_s_setprio(1);
      if (k + 1 < d.c) stage_store(k + 1, sreg);
    }

    // ---- StatePassing (Eq. 6) in registers; publish H_k for the next ChunkScan1 ----
    const int qd = s_qd[o];
    const v2s qd2 = {(short)qd, (short)qd};
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int p = 16 * (pt0 + j) + l16;
      if (k == 0 && !has_init) {
        H8[j] = pack_pairs(S8a[j], S8b[j]);
      } else {
        const v2s r01 = rsh7_pair(qd2, unpack_pair(H8[j], 0x010c000cu));
        const v2s r23 = rsh7_pair(qd2, unpack_pair(H8[j], 0x030c020cu));
        H8[j] = pack_pairs(sat127_pair(S8a[j] + r01), sat127_pair(S8b[j] + r23));
      }
      *(uint32_t*)&h8w[bsw<NS>(p, 16 * nt_own + 4 * lg)] = H8[j];
      const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kHP + p) * NS + 16 * nt_own + 4 * lg;
      if (TAPS && a.tap_s8) *(uint32_t*)(a.tap_s8 + so) = pack_pairs(S8a[j], S8b[j]);
      if (TAPS && a.tap_passed) *(uint32_t*)(a.tap_passed + so) = H8[j];
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (a.final_state) {
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int p = 16 * (pt0 + j) + l16;
      *(uint32_t*)(a.final_state + (bh_ * kHP + p) * NS + 16 * nt_own + 4 * lg) = H8[j];
    }
  }
}


template <int DT, int LC, int NS, bool TAPS>
__global__ __launch_bounds__(kCompT, 1) void k_fused_i8v2(I8Args a) {
  __shared__ __attribute__((aligned(16))) u16 s_x[2 * LC * kHP];
  __shared__ __attribute__((aligned(16))) int8_t s_qx[2 * LC * kHP];
  __shared__ __attribute__((aligned(16))) int8_t s_h8[2 * kHP * NS];
  __shared__ __attribute__((aligned(16))) float s_va[2 * LC];
  __shared__ __attribute__((aligned(16))) float s_vb[2 * LC];
  __shared__ __attribute__((aligned(16))) float s_vw[kCompW * LC];
  __shared__ __attribute__((aligned(16))) float s_ss[3 * kHP];
  __shared__ int s_qd[2];
  const int64_t bid = blockIdx.x;
  if (bid < a.nfull)
    fused_i8_v2<DT, LC, NS, 4, TAPS>(a, bid, s_x, s_qx, s_h8, s_va, s_vb, s_vw, s_ss, s_qd);
  else
    fused_i8_v2<DT, LC, NS, 2, TAPS>(a, bid - a.nfull, s_x, s_qx, s_h8, s_va, s_vb, s_vw, s_ss, s_qd);
}

template <int DT, int LC, int NS>
hipError_t launch_i8v2(const Dims& d, const void* X, const void* dt, const float* A, const void* B,
                       const void* C, const float* D, const ScalePtrs& sc, void* Y, const void* init,
                       void* final_state, void* ws, int8_t* tap_qxs, int32_t* tap_s32, int8_t* tap_s8,
                       int8_t* tap_passed, hipStream_t st) {
  const size_t Lp = (size_t)d.c * LC;
  const size_t bkg = (size_t)d.B * d.c * d.G;
  char* w = (char*)ws;
  int8_t* qC = (int8_t*)w;
  w += ws_align((size_t)d.B * Lp * d.G * NS);
  int8_t* qbt = (int8_t*)w;
  w += ws_align(bkg * NS * LC);
  u16* cbf = (u16*)w;
  w += ws_align(bkg * cb_frags(LC) * 1024);
  const size_t cs = (size_t)d.B * d.H * d.c * LC * sizeof(float);
  float* dAcs = (float*)w;
  w += ws_align(cs);
  float* lut = (float*)w;
  w += ws_align(cs);
  uint8_t* qd = (uint8_t*)w;

  // ChunkCumsum blocks and the B/C + ChunkBMM blocks side by side in one launch
  const int64_t ncs = (int64_t)d.c * d.B * ((d.H + kCsHeads - 1) / kCsHeads);
  // block kind by the number of units (measured: 8 units favour pairs of row
  // tiles, 64 units halves, 256 and 512 units one block per unit; quarters of
  // 64 units were slower: with the cumsum blocks the launch no longer fits
  // the CUs at once)
  const int cb_kind = bkg < 32 ? kCbPairs : (2 * (int64_t)bkg <= cu_count() ? kCbHalves : kCbUnit);
  const int64_t ncb = (int64_t)bkg * (cb_kind == kCbUnit ? 1 : cb_kind == kCbHalves ? 2 : LC / 32);
  if (ncs + ncb >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_prep_cb<DT, LC, NS>), dim3((unsigned)(ncs + ncb)), dim3(kPrepT), 0, st, d, dt, A, dAcs, lut,
                     qd, B, C, sc.inv_B, sc.inv_C, sc.s_B, sc.s_C, qC, qbt, cbf, (int)ncs, cb_kind);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  if (use_chunked_i8(d)) {
    int8_t* states = (int8_t*)((char*)ws + i8_states_offset(d));
    return launch_chunked_i8(d, DT, X, dt, qC, qbt, cbf, dAcs, lut, qd, D, sc, Y, init, final_state, states, tap_qxs,
                             tap_s32, tap_s8, tap_passed, st);
  }
  const SplitPlan p = split_plan(d);
  const I8Args fa{d, X, dt, qC, qbt, cbf, dAcs, lut, qd, D, sc, Y, (const int8_t*)init, (int8_t*)final_state,
                  tap_qxs, tap_s32, tap_s8, tap_passed, p.nfull, p.unit_map, p.half_il};
  const int64_t blocks = p.nfull + 2 * p.nhalf;
  if (blocks == 0) return hipSuccess;
  if (tap_qxs || tap_s32 || tap_s8 || tap_passed)
    hipLaunchKernelGGL((k_fused_i8v2<DT, LC, NS, true>), dim3((unsigned)blocks), dim3(kCompT), 0, st, fa);
  else
    hipLaunchKernelGGL((k_fused_i8v2<DT, LC, NS, false>), dim3((unsigned)blocks), dim3(kCompT), 0, st, fa);
  return hipGetLastError();
}

}  // namespace

// Workspace: Q(C) rows, Q(B)^T fragments, CB' fragments, dAcs, LUT_state,
// Q(Decay), then (chunk-parallel schedule) the int8 states [B, c, H, P, N].
size_t i8_states_offset(const Dims& d) {
  const size_t Lp = (size_t)d.c * d.l;
  const size_t bkg = (size_t)d.B * d.c * d.G;
  const size_t cs = (size_t)d.B * d.H * d.c * d.l * sizeof(float);
  return ws_align((size_t)d.B * Lp * d.G * d.N) + ws_align(bkg * d.N * d.l) +
         ws_align(bkg * cb_frags(d.l) * 1024) + 2 * ws_align(cs) + ws_align((size_t)d.B * d.H * d.c);
}

// The chunk-parallel schedule serves layers whose heads cannot fill the chip
// with one workgroup per head (measured: at B*H = 64 and 80 on 256 CUs it is
// 2-5x faster; at B*H = 512 and 640 the head-persistent kernel is 1.2x faster).
bool use_chunked_i8(const Dims& d) {
  if (d.sched == kSchedHead) return false;
  if (d.sched == kSchedChunk) return true;
  return d.B * d.H < 2 * (int64_t)cu_count();
}

size_t fused_i8_workspace_bytes(const Dims& d) {
  return i8_states_offset(d) + (use_chunked_i8(d) ? ws_align(chunked_i8_states_bytes(d)) : 0);
}

hipError_t launch_forward_i8(const Dims& d, int dtype, const void* X, const void* dt, const float* A,
                             const void* B, const void* C, const float* D, const ScalePtrs& sc, void* Y,
                             const void* init, void* final_state, void* ws, int8_t* tap_qxs, int32_t* tap_s32,
                             int8_t* tap_s8, int8_t* tap_passed, hipStream_t st) {
#define SSD_I8_CASE(DTV, LCV, NSV)                                                                          \
  if (dtype == DTV && d.l == LCV && d.N == NSV)                                                             \
    return launch_i8v2<DTV, LCV, NSV>(d, X, dt, A, B, C, D, sc, Y, init, final_state, ws, tap_qxs, tap_s32, \
                                      tap_s8, tap_passed, st);
  SSD_I8_CASE(DT_F16, 256, 128)
  SSD_I8_CASE(DT_F16, 256, 64)
  SSD_I8_CASE(DT_F16, 128, 128)
  SSD_I8_CASE(DT_F16, 128, 64)
  SSD_I8_CASE(DT_BF16, 256, 128)
  SSD_I8_CASE(DT_BF16, 256, 64)
  SSD_I8_CASE(DT_BF16, 128, 128)
  SSD_I8_CASE(DT_BF16, 128, 64)
#undef SSD_I8_CASE
  return hipErrorNotSupported;
}

}  // namespace ssd
