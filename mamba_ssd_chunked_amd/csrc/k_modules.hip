// Module kernels of the SSD chunked forward: QuantizeBC, ChunkCumsum,
// ChunkState, StatePassing, ChunkBMM, ChunkScan (float and INT8 paths).
//
// Method: "SSDi8: Accurate and Efficient 8-bit Quantization for State Space
// Duality" (paper notes page, ICLR 2026), "Overall framework" and "Key
// designs 1-3"; the float path is the plain chunked algebra of the selective
// state-space recurrence.
#include "ssd_cumsum.hpp"
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// ---------------------------------------------------------------------------
// QuantizeBC: Q(B), Q(C) once per group at SSD entry ("Overall framework",
// "Key design 3"). Each thread converts 8 consecutive elements (same group).
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_quantize_bc(const void* __restrict__ B,
                                                     const void* __restrict__ C,
                                                     const float* __restrict__ inv_B,
                                                     const float* __restrict__ inv_C,
                                                     int8_t* __restrict__ qB,
                                                     int8_t* __restrict__ qC, int64_t nvec,
                                                     int N, int G) {
  for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = v * 8;
    const int g = (int)((e0 / N) % G);
    const float ib = inv_B[g], ic = inv_C[g];
    float xb[8], xc[8];
    ld8_f<DT>(B, e0, xb);
    ld8_f<DT>(C, e0, xc);
    uint2 ob, oc;
    ob.x = pack4(q_sat(xb[0] * ib, 127.f), q_sat(xb[1] * ib, 127.f), q_sat(xb[2] * ib, 127.f),
                 q_sat(xb[3] * ib, 127.f));
    ob.y = pack4(q_sat(xb[4] * ib, 127.f), q_sat(xb[5] * ib, 127.f), q_sat(xb[6] * ib, 127.f),
                 q_sat(xb[7] * ib, 127.f));
    oc.x = pack4(q_sat(xc[0] * ic, 127.f), q_sat(xc[1] * ic, 127.f), q_sat(xc[2] * ic, 127.f),
                 q_sat(xc[3] * ic, 127.f));
    oc.y = pack4(q_sat(xc[4] * ic, 127.f), q_sat(xc[5] * ic, 127.f), q_sat(xc[6] * ic, 127.f),
                 q_sat(xc[7] * ic, 127.f));
    *(uint2*)(qB + e0) = ob;
    *(uint2*)(qC + e0) = oc;
  }
}

// ---------------------------------------------------------------------------
// Q(X) of the Table 5 "Q(X) only" row: x quantised once per (h, p) with its own
// static step, sat127(RHAZ(fl32(x * inv_Xq[h,p]))). Each thread converts 8
// consecutive elements (one head, 8 consecutive p).
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(256) void k_quantize_x(const void* __restrict__ X,
                                                    const float* __restrict__ inv_Xq,
                                                    int8_t* __restrict__ qx, int64_t nvec, int HP) {
  for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nvec;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = v * 8;
    const int hp0 = (int)(e0 % HP);
    float xv[8];
    ld8_f<DT>(X, e0, xv);
    int q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = q_sat(xv[j] * inv_Xq[hp0 + j], 127.f);
    *(uint2*)(qx + e0) = make_uint2(pack4(q[0], q[1], q[2], q[3]), pack4(q[4], q[5], q[6], q[7]));
  }
}

// ---------------------------------------------------------------------------
// ChunkCumsum (block body in ssd_cumsum.hpp): grid (c, B, ceil(H / kCsHeads)).
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kCsThreads) void k_chunk_cumsum(const void* __restrict__ dt,
                                                      const float* __restrict__ A,
                                                      float* __restrict__ dAcs,
                                                      float* __restrict__ lut,
                                                      uint8_t* __restrict__ qdecay, Dims d) {
  __shared__ CsLds cs;
  chunk_cumsum_block<DT>(dt, A, dAcs, lut, qdecay, d, blockIdx.x, blockIdx.y, blockIdx.z, cs);
}

// ---------------------------------------------------------------------------
// ChunkState ("Key design 1", Eq. 4 via the reconstruction). One workgroup of
// four waves per (h, k, b). The sequence axis s (the GEMM's K) is staged in
// blocks of 64 through LDS, transposed so each lane reads 16 contiguous bytes.
// Output tiles (16 x 16 over P x N) are spread over the four waves.
// ---------------------------------------------------------------------------
constexpr int kStK = 64;  // s per staged block

// MODE (ssd_launch.hpp): kModeFloat, kModeInt8 (S8 requantised, "Key design 2"),
// kModeQx (X read as int8 Q(X) times its step sx[h,p]; float otherwise) and
// kModeRecon (S32 on INT8 as in kModeInt8, dequantised to fp32 with
// sx[h,p] * sb[g] instead of requantised).
template <int DT, int MODE>
__global__ __launch_bounds__(256) void k_chunk_state(Dims d, const void* __restrict__ X,
                                                     const float* __restrict__ lut,
                                                     const void* __restrict__ Bq,
                                                     const float* __restrict__ inv_X,
                                                     const float* __restrict__ M_req,
                                                     const float* __restrict__ sx,
                                                     const float* __restrict__ sb,
                                                     void* __restrict__ states,
                                                     int8_t* __restrict__ tap_qxs,
                                                     int32_t* __restrict__ tap_s32) {
  constexpr bool INT8 = MODE == kModeInt8 || MODE == kModeRecon;
  typedef typename Store<DT>::T T;
  constexpr int PAD = INT8 ? 16 : (16 / (int)sizeof(T));
  typedef typename std::conditional<INT8, int8_t, T>::type E;
  __shared__ __attribute__((aligned(16))) E sX[64][kStK + PAD];
  __shared__ __attribute__((aligned(16))) E sB[128][kStK + PAD];
  // low bf16 half of X_scaled (bf16 float path only, see FragC)
  constexpr bool kSplit = !INT8 && DT == DT_BF16;
  __shared__ __attribute__((aligned(16))) E sXlo[kSplit ? 64 : 1][kSplit ? kStK + PAD : 1];

  const int h = blockIdx.x, k = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int g = h / d.hpg;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int P = d.P, N = d.N, H = d.H;
  const int ntN = N / 16, ntiles = (P / 16) * ntN;
  const int64_t lut0 = ((b * H + h) * d.c + k) * (int64_t)d.l;

  typedef typename std::conditional<INT8, v4i, v4f>::type Acc;
  Acc acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = Acc{0, 0, 0, 0};

  for (int s0 = 0; s0 < d.l; s0 += kStK) {
    // stage X_scaled (quantised on the INT8 path) transposed: sX[p][s]
    for (int item = tid; item < kStK * (P / 8); item += 256) {
      const int s = item / (P / 8), p0 = (item % (P / 8)) * 8;
      const int64_t t = (int64_t)k * d.l + s0 + s;
      float xv[8];
      if (t < d.L) {
        const int64_t xo = ((b * d.L + t) * H + h) * (int64_t)P + p0;
        if constexpr (MODE == kModeQx) {
          const uint2 q = *(const uint2*)((const int8_t*)X + xo);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            xv[j] = (float)byte_s(j < 4 ? q.x : q.y, j % 4) * sx[h * P + p0 + j];
        } else {
          ld8_f<DT>(X, xo, xv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = 0.f;
      }
      const float lv = lut[lut0 + s0 + s];
      if constexpr (INT8) {
        int q[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xs = lv * xv[j];                 // fl32(LUT * x)
          q[j] = q_sat(xs * inv_X[h * P + p0 + j], 127.f);
          sX[p0 + j][s] = (int8_t)q[j];
        }
        if (tap_qxs && t < d.L) {
          uint2 o;
          o.x = pack4(q[0], q[1], q[2], q[3]);
          o.y = pack4(q[4], q[5], q[6], q[7]);
          *(uint2*)(tap_qxs + ((b * d.L + t) * H + h) * (int64_t)P + p0) = o;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xs = lv * xv[j];
          const T hi = to_store<DT>(xs);
          sX[p0 + j][s] = hi;
          if constexpr (kSplit) sXlo[p0 + j][s] = to_store<DT>(xs - Store<DT>::to_f(hi));
        }
      }
    }
    // stage B (int8 Q(B) or input dtype) transposed: sB[n][s]
    if constexpr (INT8) {
      for (int item = tid; item < kStK * (N / 16); item += 256) {
        const int s = item / (N / 16), n0 = (item % (N / 16)) * 16;
        const int64_t t = (int64_t)k * d.l + s0 + s;
        uint4 v = {0, 0, 0, 0};
        if (t < d.L) v = *(const uint4*)((const int8_t*)Bq + ((b * d.L + t) * d.G + g) * (int64_t)N + n0);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 16; ++j) sB[n0 + j][s] = (int8_t)byte_s(wv[j / 4], j % 4);
      }
    } else {
      for (int item = tid; item < kStK * (N / 8); item += 256) {
        const int s = item / (N / 8), n0 = (item % (N / 8)) * 8;
        const int64_t t = (int64_t)k * d.l + s0 + s;
        float bv[8];
        if (t < d.L) {
          ld8_f<DT>(Bq, ((b * d.L + t) * d.G + g) * (int64_t)N + n0, bv);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) bv[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) sB[n0 + j][s] = to_store<DT>(bv[j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tile = w + 4 * j;
      if (tile < ntiles) {
        const int pt = tile / ntN, nt = tile % ntN;
        if constexpr (INT8) {
          const v4i a = *(const v4i*)&sX[pt * 16 + (lane & 15)][(lane >> 4) * 16];
          const v4i bb = *(const v4i*)&sB[nt * 16 + (lane & 15)][(lane >> 4) * 16];
          acc[j] = mma_i8(a, bb, acc[j]);
        } else {
#pragma unroll
          for (int kk = 0; kk < kStK; kk += 32) {
            FragF<DT> a, bb;
            lds_frag8<DT>(&sX[pt * 16 + (lane & 15)][kk + (lane >> 4) * 8], a);
            lds_frag8<DT>(&sB[nt * 16 + (lane & 15)][kk + (lane >> 4) * 8], bb);
            acc[j] = FragF<DT>::mma(a, bb, acc[j]);
            if constexpr (kSplit) {
              lds_frag8<DT>(&sXlo[pt * 16 + (lane & 15)][kk + (lane >> 4) * 8], a);
              acc[j] = FragF<DT>::mma(a, bb, acc[j]);
            }
          }
        }
      }
    }
    __syncthreads();
  }
  // epilogue: requantise in registers ("Key design 2") or store fp32
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tile = w + 4 * j;
    if (tile < ntiles) {
      const int pt = tile / ntN, nt = tile % ntN;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = pt * 16 + 4 * (lane >> 4) + r, n = nt * 16 + (lane & 15);
        const int64_t off = (((b * d.c + k) * H + h) * (int64_t)P + p) * N + n;
        if constexpr (MODE == kModeInt8) {
          const int v = acc[j][r];
          if (tap_s32) tap_s32[off] = v;
          ((int8_t*)states)[off] = (int8_t)q_sat((float)v * M_req[h * P + p], 127.f);
        } else if constexpr (MODE == kModeRecon) {
          ((float*)states)[off] = (float)acc[j][r] * (sx[h * P + p] * sb[g]);
        } else {
          ((float*)states)[off] = acc[j][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// StatePassing (Eq. 6), element-parallel over (b, h, p, n), sequential over
// chunks.
// ---------------------------------------------------------------------------

// INT8: Eq. 6 over the chunks of every (b, h, p, n) element, four elements
// (one dword) per thread, updated as int16 pairs. The chain is sequential per
// element; the loads of the next G chunks are issued before the current G are
// updated, so 2 G chunk loads per thread are in flight. Every thread issues the
// same loads and stores in every group (chunks past the end re-read and
// re-store the last chunk's slot with its final value, unchanged), so the
// compiler's in-order wait counts are exact and never wait for the prefetch.
template <int G>
__global__ __launch_bounds__(256) void k_state_passing_i8(Dims d, int8_t* __restrict__ states,
                                                          const uint8_t* __restrict__ qdecay,
                                                          const int8_t* __restrict__ init,
                                                          int8_t* __restrict__ final_state) {
  const int64_t per_b = (int64_t)d.H * d.P * d.N / 4;  // dwords per (b, chunk) slot
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= d.B * per_b) return;
  const int64_t b = e / per_b, r = e % per_b;
  const int h = (int)((r * 4) / ((int64_t)d.P * d.N));
  uint32_t* st = (uint32_t*)states;
  const int64_t slot = per_b;  // dwords per chunk slot
  const int64_t base = b * d.c * slot + r;
  // without an initial state H_0 = S_0; with one, Eq. 6 applies from chunk 0
  uint32_t prev = init ? ((const uint32_t*)init)[b * per_b + r] : st[base];
  const int64_t q0 = (b * d.H + h) * d.c;                       // this head's first Q(Decay) byte
  const int64_t qlast = ((d.B * d.H * d.c - 1) & ~(int64_t)3);  // last whole dword of the array
  const int k_begin = init ? 0 : 1;
  const int ngroups = (d.c - k_begin + G - 1) / G;
  // the group's states, and its G Q(Decay) bytes from G / 4 + 1 aligned dwords
  // (addresses clamped into the array; a clamped dword only ever feeds chunks
  // past the end)
  const auto load = [&](int g, uint32_t (&v)[G], int (&q)[G]) {
    const int kg = k_begin + g * G;
#pragma unroll
    for (int j = 0; j < G; ++j) v[j] = st[base + (int64_t)min(kg + j, d.c - 1) * slot];
    const int64_t a = q0 + kg;
    const int sh = (int)(a & 3);
    uint32_t w[G / 4 + 1];
#pragma unroll
    for (int i = 0; i <= G / 4; ++i) w[i] = *(const uint32_t*)(qdecay + min((a & ~(int64_t)3) + 4 * i, qlast));
#pragma unroll
    for (int i = 0; i < G / 4; ++i) {
      const uint32_t u = __builtin_amdgcn_alignbyte(w[i + 1], w[i], (uint32_t)sh);
#pragma unroll
      for (int z = 0; z < 4; ++z) q[4 * i + z] = (int)((u >> (8 * z)) & 0xffu);
    }
  };
  const auto step = [&](int g, const uint32_t (&v)[G], const int (&q)[G]) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int kr = k_begin + g * G + j;
      const v2s qd2 = {(short)q[j], (short)q[j]};
      const v2s h01 = sat127_pair(unpack_pair(v[j], 0x010c000cu) + rsh7_pair(qd2, unpack_pair(prev, 0x010c000cu)));
      const v2s h23 = sat127_pair(unpack_pair(v[j], 0x030c020cu) + rsh7_pair(qd2, unpack_pair(prev, 0x030c020cu)));
      if (kr < d.c) prev = pack_pairs(h01, h23);
      st[base + (int64_t)min(kr, d.c - 1) * slot] = prev;
    }
  };
  uint32_t va[G], vb[G];
  int qa[G], qb[G];
  load(0, va, qa);
  for (int g = 0; g < ngroups; g += 2) {
    load(g + 1, vb, qb);
    step(g, va, qa);
    load(g + 2, va, qa);
    step(g + 1, vb, qb);
  }
  if (final_state) ((uint32_t*)final_state)[b * per_b + r] = prev;
}

__global__ __launch_bounds__(256) void k_state_passing_f(Dims d, float* __restrict__ states,
                                                         const float* __restrict__ dAcs,
                                                         const float* __restrict__ init,
                                                         float* __restrict__ final_state) {
  const int64_t per_b = (int64_t)d.H * d.P * d.N / 4;  // float4 per slot
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= d.B * per_b) return;
  const int64_t b = e / per_b, r = e % per_b;
  const int h = (int)((r * 4) / ((int64_t)d.P * d.N));
  float4* st = (float4*)states;
  const int64_t slot = per_b;
  const int64_t base = b * d.c * slot + r;
  float4 prev = init ? ((const float4*)init)[b * per_b + r] : st[base];
  const float* da = dAcs + (b * d.H + h) * (int64_t)d.c * d.l;
  for (int k0 = init ? 0 : 1; k0 < d.c; k0 += 8) {
    float4 v[8];
    float dec[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (k0 + j < d.c) {
        v[j] = st[base + (int64_t)(k0 + j) * slot];
        dec[j] = expf(da[(int64_t)(k0 + j) * d.l + d.l - 1]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (k0 + j < d.c) {
        prev.x = dec[j] * prev.x + v[j].x;
        prev.y = dec[j] * prev.y + v[j].y;
        prev.z = dec[j] * prev.z + v[j].z;
        prev.w = dec[j] * prev.w + v[j].w;
        st[base + (int64_t)(k0 + j) * slot] = prev;
      }
    }
  }
  if (final_state) ((float4*)final_state)[b * per_b + r] = prev;
}

// ---------------------------------------------------------------------------
// ChunkBMM: CB = C B^T per (g, k, b), lower-triangular 16 x 16 tiles.
// ---------------------------------------------------------------------------
template <int DT, bool INT8>
__global__ __launch_bounds__(256) void k_chunk_bmm(Dims d, const void* __restrict__ Cq,
                                                   const void* __restrict__ Bq,
                                                   void* __restrict__ CB) {
  const int g = blockIdx.x, k = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int lane = lane_id(), w = wave_id();
  const int nt = d.l / 16, N = d.N;
  const int64_t cb0 = ((b * d.c + k) * d.G + g) * (int64_t)d.l * d.l;
  for (int tile = w; tile < nt * nt; tile += 4) {
    const int it = tile / nt, jt = tile % nt;
    const int i = it * 16 + (lane & 15), j = jt * 16 + (lane & 15);
    const int64_t ti = (int64_t)k * d.l + i, tj = (int64_t)k * d.l + j;
    typedef typename std::conditional<INT8, v4i, v4f>::type Acc;
    Acc acc = Acc{0, 0, 0, 0};
    if (jt <= it) {
      if constexpr (INT8) {
        for (int kk = 0; kk < N; kk += 64) {
          v4i a = {0, 0, 0, 0}, bb = {0, 0, 0, 0};
          const int n = kk + (lane >> 4) * 16;
          // K lanes past N (N < 64) contribute zeros
          if (ti < d.L && n < N) a = *(const v4i*)((const int8_t*)Cq + ((b * d.L + ti) * d.G + g) * (int64_t)N + n);
          if (tj < d.L && n < N) bb = *(const v4i*)((const int8_t*)Bq + ((b * d.L + tj) * d.G + g) * (int64_t)N + n);
          acc = mma_i8(a, bb, acc);
        }
      } else {
        for (int kk = 0; kk < N; kk += 32) {
          FragF<DT> a, bb;
          const int n = kk + (lane >> 4) * 8;
          if (ti < d.L && n < N) glb_frag8<DT>(Cq, ((b * d.L + ti) * d.G + g) * (int64_t)N + n, a); else a.zero();
          if (tj < d.L && n < N) glb_frag8<DT>(Bq, ((b * d.L + tj) * d.G + g) * (int64_t)N + n, bb); else bb.zero();
          acc = FragF<DT>::mma(a, bb, acc);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ii = it * 16 + 4 * (lane >> 4) + r, jj = jt * 16 + (lane & 15);
      const int64_t off = cb0 + (int64_t)ii * d.l + jj;
      if constexpr (INT8) {
        ((int32_t*)CB)[off] = jj <= ii ? acc[r] : 0;
      } else {
        ((float*)CB)[off] = jj <= ii ? acc[r] : 0.f;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// ChunkScan1 + ChunkScan2 + D skip. One workgroup per (h, k, b); wave w owns
// row tiles w, w+4, w+8, w+12 (balanced under the causal mask) and all P/16
// column tiles. x is staged transposed in LDS in the compute type.
// ---------------------------------------------------------------------------
// MODE: kModeFloat, kModeInt8 (Scan1 on the int8 passed states and Q(C), Scan2
// on the int32 CB with s_C s_B folded into its weights), kModeQx (float, X read
// as int8 Q(X) times its step sx[h,p]) and kModeRecon (Scan1 on INT8: the fp32
// passed states are quantised with the state step s_S as they are read and
// contracted with Q(C); Scan2 on the fp32 CB of the unquantised B and C).
template <int DT, int MODE>
__global__ __launch_bounds__(256) void k_chunk_scan(Dims d, const void* __restrict__ X,
                                                    const void* __restrict__ dt,
                                                    const float* __restrict__ dAcs,
                                                    const void* __restrict__ Cq,
                                                    const void* __restrict__ CB,
                                                    const void* __restrict__ states,
                                                    const void* __restrict__ init,
                                                    const float* __restrict__ D,
                                                    const float* __restrict__ s_C,
                                                    const float* __restrict__ s_B,
                                                    const float* __restrict__ s_S,
                                                    const float* __restrict__ sx,
                                                    void* __restrict__ Y) {
  constexpr bool INT8 = MODE == kModeInt8;            // int32 CB with folded scales
  constexpr bool SCAN1_I8 = MODE == kModeInt8 || MODE == kModeRecon;
  typedef typename Store<DT>::T T;
  constexpr int PAD = 16 / (int)sizeof(T);
  __shared__ __attribute__((aligned(16))) T sxT[64][256 + PAD];
  __shared__ float sdA[256];
  __shared__ float sdt[256];

  const int h = blockIdx.x, k = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int g = h / d.hpg;
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  const int P = d.P, N = d.N, H = d.H, l = d.l;
  const int RT = l / 16, PT = P / 16;
  const int64_t t0 = (int64_t)k * l;

  for (int item = tid; item < l * (P / 8); item += 256) {
    const int s = item / (P / 8), p0 = (item % (P / 8)) * 8;
    float xv[8];
    if (t0 + s < d.L) {
      const int64_t xo = ((b * d.L + t0 + s) * H + h) * (int64_t)P + p0;
      if constexpr (MODE == kModeQx) {
        const uint2 q = *(const uint2*)((const int8_t*)X + xo);
#pragma unroll
        for (int j = 0; j < 8; ++j) xv[j] = (float)byte_s(j < 4 ? q.x : q.y, j % 4) * sx[h * P + p0 + j];
      } else {
        ld8_f<DT>(X, xo, xv);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) xv[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) sxT[p0 + j][s] = to_store<DT>(xv[j]);
  }
  for (int s = tid; s < l; s += 256) {
    sdA[s] = dAcs[((b * H + h) * d.c + k) * (int64_t)l + s];
    sdt[s] = (t0 + s < d.L) ? ld_f<DT>(dt, (b * d.L + t0 + s) * H + h) : 0.f;
  }
  __syncthreads();

  const float cbscale = INT8 ? s_C[g] * s_B[g] : 1.f;
  const int64_t cb0 = ((b * d.c + k) * d.G + g) * (int64_t)l * l;
  const float Dh = D[h];

  for (int ri = 0; ri < 4; ++ri) {
    const int it = w + 4 * ri;
    if (it >= RT) break;
    v4f acc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = v4f{0, 0, 0, 0};
    // ChunkScan2 (intra-chunk)
    const int s = it * 16 + (lane & 15);
    const float dAs = sdA[s];
    const int nk = ((it + 1) * 16 + 31) / 32;
    for (int kb = 0; kb < nk; ++kb) {
      FragC<DT> a;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sp = kb * 32 + (lane >> 4) * 8 + e;
        float wv = 0.f;
        if (sp <= s) {
          const float cbv = INT8 ? (float)((const int32_t*)CB)[cb0 + (int64_t)s * l + sp]
                                 : ((const float*)CB)[cb0 + (int64_t)s * l + sp];
          wv = cbv * cbscale * expf(dAs - sdA[sp]) * sdt[sp];
        }
        a.set(e, wv);
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        if (pt < PT) {
          FragF<DT> bx;
          lds_frag8<DT>(&sxT[pt * 16 + (lane & 15)][kb * 32 + (lane >> 4) * 8], bx);
          acc[pt] = mma_ca<DT>(a, bx, acc[pt]);
        }
      }
    }
    // ChunkScan1 (inter-chunk): the passed state of chunk k - 1, or the initial
    // state for chunk 0 when one is given
    v4f yoff[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) yoff[pt] = v4f{0, 0, 0, 0};
    const bool has_prev = k > 0 || init != nullptr;
    const void* const sprev = k > 0 ? states : init;
    if (has_prev) {
      const int64_t st0 = (k > 0 ? ((b * d.c + (k - 1)) * H + h) : (b * H + h)) * (int64_t)P * N;
      const int64_t ts = t0 + s;
      if constexpr (SCAN1_I8) {
        v4i acc1[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc1[pt] = v4i{0, 0, 0, 0};
        for (int kk = 0; kk < N; kk += 64) {
          const int n = kk + (lane >> 4) * 16;
          v4i a = {0, 0, 0, 0};
          if (ts < d.L && n < N) a = *(const v4i*)((const int8_t*)Cq + ((b * d.L + ts) * d.G + g) * (int64_t)N + n);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            if (pt < PT) {
              v4i hb = {0, 0, 0, 0};
              const int pr = pt * 16 + (lane & 15);
              if (n < N) {
                if constexpr (MODE == kModeRecon) {
                  // Q(H) = sat(RHAZ(H / s_S[h,p])) of the fp32 passed state
                  const float* hp = (const float*)sprev + st0 + (int64_t)pr * N + n;
                  const float sS = s_S[h * P + pr];
                  int q[16];
#pragma unroll
                  for (int e = 0; e < 16; ++e) q[e] = q_sat(hp[e] / sS, 127.f);
#pragma unroll
                  for (int e = 0; e < 4; ++e) hb[e] = (int)pack4(q[4 * e], q[4 * e + 1], q[4 * e + 2], q[4 * e + 3]);
                } else {
                  hb = *(const v4i*)((const int8_t*)sprev + st0 + (int64_t)pr * N + n);
                }
              }
              acc1[pt] = mma_i8(a, hb, acc1[pt]);
            }
          }
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) yoff[pt][r] = (float)acc1[pt][r];
        }
      } else {
        for (int kk = 0; kk < N; kk += 32) {
          const int n = kk + (lane >> 4) * 8;
          FragF<DT> a;
          if (ts < d.L && n < N) glb_frag8<DT>(Cq, ((b * d.L + ts) * d.G + g) * (int64_t)N + n, a); else a.zero();
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            if (pt < PT) {
              FragC<DT> hb;
              hb.zero();
              if (n < N) {
                const float* hp = (const float*)sprev + st0 + (int64_t)(pt * 16 + (lane & 15)) * N + n;
#pragma unroll
                for (int e = 0; e < 8; ++e) hb.set(e, hp[e]);
              }
              yoff[pt] = mma_cb<DT>(a, hb, yoff[pt]);
            }
          }
        }
      }
    }
    // epilogue
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      if (pt < PT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sr = it * 16 + 4 * (lane >> 4) + r;
          const int p = pt * 16 + (lane & 15);
          const float xv = (float)Store<DT>::to_f(sxT[p][sr]);
          float y = acc[pt][r] + Dh * xv;
          if (has_prev) {
            float f = expf(sdA[sr]);
            if (SCAN1_I8) f *= s_C[g] * s_S[h * P + p];
            y += yoff[pt][r] * f;
          }
          const int64_t t = t0 + sr;
          if (t < d.L) ((T*)Y)[((b * d.L + t) * H + h) * (int64_t)P + p] = to_store<DT>(y);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#define SSD_DISPATCH_DT(dtype, FN) \
  switch (dtype) {                 \
    case DT_F32: FN(DT_F32); break; \
    case DT_F16: FN(DT_F16); break; \
    case DT_BF16: FN(DT_BF16); break; \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_quantize_bc(const Dims& d, int dtype, const void* B, const void* C,
                              const float* inv_B, const float* inv_C, int8_t* qB, int8_t* qC,
                              hipStream_t st) {
  const int64_t nvec = d.B * d.L * d.G * (int64_t)d.N / 8;
  const int64_t want = (nvec + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? (want > 0 ? want : 1) : 8192);
#define L_(DT_) hipLaunchKernelGGL(k_quantize_bc<DT_>, dim3(grid), dim3(256), 0, st, B, C, inv_B, inv_C, qB, qC, nvec, d.N, d.G)
  SSD_DISPATCH_DT(dtype, L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_quantize_x(const Dims& d, int dtype, const void* X, const float* inv_Xq,
                             int8_t* qx, hipStream_t st) {
  const int64_t nvec = d.B * d.L * d.H * (int64_t)d.P / 8;
  const int64_t want = (nvec + 255) / 256;
  const unsigned grid = (unsigned)(want < 8192 ? (want > 0 ? want : 1) : 8192);
#define L_(DT_) hipLaunchKernelGGL(k_quantize_x<DT_>, dim3(grid), dim3(256), 0, st, X, inv_Xq, qx, nvec, d.H * d.P)
  SSD_DISPATCH_DT(dtype, L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_chunk_cumsum(const Dims& d, int dtype, const void* dt, const float* A,
                               float* dAcs, float* lut, uint8_t* qdecay, hipStream_t st) {
  const dim3 grid(d.c, (unsigned)d.B, (d.H + kCsHeads - 1) / kCsHeads);
#define L_(DT_) hipLaunchKernelGGL(k_chunk_cumsum<DT_>, grid, dim3(kCsThreads), 0, st, dt, A, dAcs, lut, qdecay, d)
  SSD_DISPATCH_DT(dtype, L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_chunk_state(const Dims& d, int dtype, int mode, const void* X,
                              const float* lut, const void* Bq, const float* inv_X,
                              const float* M_req, const float* sx, const float* sb, void* states,
                              int8_t* tap_qxs, int32_t* tap_s32, hipStream_t st) {
  const dim3 grid(d.H, d.c, (unsigned)d.B);
#define L_(DT_) hipLaunchKernelGGL((k_chunk_state<DT_, M_>), grid, dim3(256), 0, st, d, X, lut, Bq, inv_X, M_req, sx, sb, states, tap_qxs, tap_s32)
  switch (mode) {
    case kModeFloat: {
      constexpr int M_ = kModeFloat;
      SSD_DISPATCH_DT(dtype, L_)
      break;
    }
    case kModeInt8: {
      constexpr int M_ = kModeInt8;
      SSD_DISPATCH_DT(dtype, L_)
      break;
    }
    case kModeQx: {
      constexpr int M_ = kModeQx;
      SSD_DISPATCH_DT(dtype, L_)
      break;
    }
    case kModeRecon: {
      constexpr int M_ = kModeRecon;
      SSD_DISPATCH_DT(dtype, L_)
      break;
    }
    default: return hipErrorInvalidValue;
  }
#undef L_
  return hipGetLastError();
}

hipError_t launch_state_passing(const Dims& d, bool int8, void* states, const float* dAcs,
                                const uint8_t* qdecay, const void* init, void* final_state,
                                hipStream_t st) {
  const int64_t n = d.B * (int64_t)d.H * d.P * d.N / 4;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (int8) {
    // short sequences take short groups (less redundant tail)
    if (d.c > 32)
      hipLaunchKernelGGL(k_state_passing_i8<16>, dim3(grid), dim3(256), 0, st, d, (int8_t*)states, qdecay,
                         (const int8_t*)init, (int8_t*)final_state);
    else
      hipLaunchKernelGGL(k_state_passing_i8<4>, dim3(grid), dim3(256), 0, st, d, (int8_t*)states, qdecay,
                         (const int8_t*)init, (int8_t*)final_state);
  } else {
    hipLaunchKernelGGL(k_state_passing_f, dim3(grid), dim3(256), 0, st, d, (float*)states, dAcs,
                       (const float*)init, (float*)final_state);
  }
  return hipGetLastError();
}

hipError_t launch_chunk_bmm(const Dims& d, int dtype, bool int8, const void* Cq,
                            const void* Bq, void* CB, hipStream_t st) {
  const dim3 grid(d.G, d.c, (unsigned)d.B);
  if (int8) {
    hipLaunchKernelGGL((k_chunk_bmm<DT_F16, true>), grid, dim3(256), 0, st, d, Cq, Bq, CB);
  } else {
#define L_(DT_) hipLaunchKernelGGL((k_chunk_bmm<DT_, false>), grid, dim3(256), 0, st, d, Cq, Bq, CB)
    SSD_DISPATCH_DT(dtype, L_)
#undef L_
  }
  return hipGetLastError();
}

hipError_t launch_chunk_scan(const Dims& d, int dtype, int mode, const void* X, const void* dt,
                             const float* dAcs, const void* Cq, const void* CB,
                             const void* states, const void* init, const float* D,
                             const float* s_C, const float* s_B, const float* s_S, const float* sx,
                             void* Y, hipStream_t st) {
  const dim3 grid(d.H, d.c, (unsigned)d.B);
#define L_(DT_) hipLaunchKernelGGL((k_chunk_scan<DT_, M_>), grid, dim3(256), 0, st, d, X, dt, dAcs, Cq, CB, states, init, D, s_C, s_B, s_S, sx, Y)
  switch (mode) {
    case kModeFloat: {
      constexpr int M_ = kModeFloat;
      SSD_DISPATCH_DT(dtype, L_)
      break;
    }
    case kModeInt8: {
      constexpr int M_ = kModeInt8;
      SSD_DISPATCH_DT(dtype, L_)
      break;
    }
    case kModeQx: {
      constexpr int M_ = kModeQx;
      SSD_DISPATCH_DT(dtype, L_)
      break;
    }
    case kModeRecon: {
      constexpr int M_ = kModeRecon;
      SSD_DISPATCH_DT(dtype, L_)
      break;
    }
    default: return hipErrorInvalidValue;
  }
#undef L_
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// zero fill (16 bytes per thread, grid-stride)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_zero_fill(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, 4096);
  hipLaunchKernelGGL(k_zero_fill, dim3((unsigned)blocks), dim3(256), 0, st, (uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace ssd
