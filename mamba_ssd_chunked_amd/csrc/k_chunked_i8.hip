// Chunk-parallel schedule of the fused INT8 forward ("SSDi8" notes page,
// "Overall framework": L = c l chunks and the five modules). Where the heads are
// too few to occupy the chip with one workgroup per head (a walk over its
// chunks), every (batch, head, chunk) gets its own workgroups:
//
//   k_cstate_i8   Q(Xs) and ChunkState S32 -> S8 per (batch, chunk, head),
//                 written to the int8 states [B, c, H, P, N];
//   StatePassing  Eq. 6 in chunk order over the states in place (the module
//                 kernel; the rounding shift is not associative, so the chain
//                 stays sequential and bit-exact);
//   k_cscan_i8    ChunkScan1 on the passed state of chunk k - 1 plus ChunkScan2
//                 and the D skip, per (batch, chunk, head).
//
// Both per-chunk kernels read the operand fragments of the preparation launch
// (k_fused_i8.hip) and keep the LDS layouts and integer arithmetic of the
// head-persistent kernel, so every integer result is the same.
#include "ssd_device.hpp"
#include "ssd_i8_layout.hpp"
#include "ssd_launch.hpp"

namespace ssd {
namespace {

constexpr int kCT = 256;  // threads of both per-chunk kernels (four waves)

struct ChunkArgs {
  Dims d;
  const void* X;
  const void* dt;
  const int8_t* qC;
  const int8_t* qbt;
  const u16* cbf;
  const float* dAcs;
  const float* lut;
  const float* D;
  ScalePtrs sc;
  int8_t* states;      // [B, c, H, P, N]: local S8 after k_cstate_i8, passed states after StatePassing
  const int8_t* init;  // optional initial state [B, H, P, N]
  void* Y;
  int8_t* tap_qxs;
  int32_t* tap_s32;
  int8_t* tap_s8;
  int xcd_map;  // (B * c * G) % 8 == 0: the units of one XCD (see chunk_block)
};

// block -> (b, k, h). The heads of one unit (batch, chunk, group) share its
// Q(B)^T, Q(C) and CB' operands. With xcd_map, block i runs on XCD i % 8 and
// serves unit (i % 8) + 8 ((i / 8) / hpg), head (i / 8) % hpg of its group: every
// unit's heads run on one XCD, whose L2 then fetches the unit's operands once.
// Otherwise consecutive blocks are the heads of one unit (all groups of a
// (batch, chunk) in turn).
struct BKH {
  int64_t b;
  int k, h;
};
__device__ __forceinline__ BKH chunk_block(const Dims& d, int xcd_map) {
  BKH r;
  const int64_t bi = blockIdx.x;
  if (xcd_map) {
    const int64_t j = bi / 8;
    const int64_t u = bi % 8 + 8 * (j / d.hpg);  // unit = (b c + k) G + g
    const int g = (int)(u % d.G);
    const int64_t bk = u / d.G;
    r.h = g * d.hpg + (int)(j % d.hpg);
    r.k = (int)(bk % d.c);
    r.b = bk / d.c;
  } else {
    r.h = (int)(bi % d.H);
    const int64_t bk = bi / d.H;
    r.k = (int)(bk % d.c);
    r.b = bk / d.c;
  }
  return r;
}

// ===========================================================================
// k_cstate_i8: Q(X_scaled) of the chunk into LDS, then S32^T[n, p] =
// sum_s Q(B)^T[n, s] Q(Xs)[s, p] on int8 MFMA (wave w: n tiles NTW w .. + NTW - 1,
// all four p tiles), requantised to S8 ("Key design 2").
// ===========================================================================
template <int DT, int LC, int NS, bool TAPS>
__global__ __launch_bounds__(kCT) void k_cstate_i8(ChunkArgs a) {
  typedef typename Store<DT>::T T;
  constexpr int NT = NS / 16, KS = LC / 64;
  constexpr int NTW = NT / 4;         // n tiles per wave
  constexpr int NU = LC * 8 / kCT;    // 16-byte x items per thread
  __shared__ __attribute__((aligned(16))) int8_t s_qx[LC * kHP];
  const Dims& d = a.d;
  const BKH u = chunk_block(d, a.xcd_map);
  const int64_t b = u.b;
  const int k = u.k, h = u.h, H = d.H;
  const int g = h / d.hpg;
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int lane = tid & (kWave - 1);
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)k * LC;
  const int64_t bh = b * H + h;

  // the requantisation factors of this lane's p values, then this wave's
  // Q(B)^T fragments, issued first (they land during the staging)
  float mreq[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) mreq[pt] = a.sc.M_req[h * kHP + 16 * pt + l16];
  v4i qa[NTW][KS];
  {
    const char* src = (const char*)a.qbt + (((b * d.c + k) * d.G + g) * (int64_t)(NT * KS)) * 1024 + 16 * lane;
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qa[j][ks] = *(const v4i*)(src + ((NTW * w + j) * KS + ks) * 1024);
  }
  // staging: thread tid quantises x rows tid / 8 + 32 v, columns 8 (tid % 8) ..
  {
    const int c8 = tid & 7, r0 = tid >> 3;
    const int64_t lim = d.L - 1 - t0;
    const int64_t rowB = (int64_t)H * kHP * sizeof(T);
    const char* xh = (const char*)a.X + ((b * d.L + t0) * H + h) * (int64_t)kHP * sizeof(T) + 16 * c8;
    const float* lp = a.lut + (bh * d.c + k) * (int64_t)LC;
    const float4 i0 = ld_scale4(&a.sc.inv_X[h * kHP + 8 * c8]);
    const float4 i1 = ld_scale4(&a.sc.inv_X[h * kHP + 8 * c8 + 4]);
    const float ix[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
    v4i xr[NU];
    float lr[NU];
#pragma unroll
    for (int v = 0; v < NU; ++v) {
      const int s = r0 + 32 * v;
      xr[v] = __builtin_nontemporal_load((const v4i*)(xh + min((int64_t)s, lim) * rowB));
      lr[v] = lp[s];
    }
#pragma unroll
    for (int v = 0; v < NU; ++v) {
      const int s = r0 + 32 * v;
      // Q(X_scaled) = sat(RHAZ(fl32(fl32(lut * x) * inv_X))) ("Key design 1"); rows
      // past L have LUT_state 0
      float q[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t dw = (uint32_t)xr[v][j];
        const float x0 = Store<DT>::to_f(__builtin_bit_cast(T, (u16)(dw & 0xffffu)));
        const float x1 = Store<DT>::to_f(__builtin_bit_cast(T, (u16)(dw >> 16)));
        q[2 * j] = __builtin_fmaf(lr[v], x0, 0.0f) * ix[2 * j];
        q[2 * j + 1] = __builtin_fmaf(lr[v], x1, 0.0f) * ix[2 * j + 1];
      }
      const uint2 qq = make_uint2(q8x4(q[0], q[1], q[2], q[3]), q8x4(q[4], q[5], q[6], q[7]));
      *(uint2*)&s_qx[qsw_off(s, 8 * c8)] = qq;
      if (TAPS && a.tap_qxs && t0 + s < d.L)
        *(uint2*)(a.tap_qxs + ((b * d.L + t0 + s) * H + h) * (int64_t)kHP + 8 * c8) = qq;
    }
  }
  __syncthreads();

  // ChunkState: B operand Q(Xs)[s, p] of p tile pt by transposing reads (rows
  // 16 lg + (l16 >> 1) + 64 ks + 8 half)
  v4i acc[NTW][4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    v4i bq[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int off = qsw_off(16 * lg + (l16 >> 1), 16 * pt + 8 * (l16 & 1)) + (64 * ks) * kHP;
      const v2i_t lo = ldtr8(s_qx + off);
      const v2i_t hi = ldtr8(s_qx + off + 8 * kHP);
      bq[pt] = v4i{lo.x, lo.y, hi.x, hi.y};
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[j][pt] = mma_i8(qa[j][ks], bq[pt], ks == 0 ? v4i{0, 0, 0, 0} : acc[j][pt]);
  }
  // requantise (lane: p = 16 pt + l16, n = 16 nt + 4 lg + r); the block's S8
  // tile [P][N] is contiguous in the states, so it is gathered in LDS (over
  // the Q(Xs) tile, once every wave is done with it) and leaves as whole lines
  // (measured on the 64K-token layer: 240 -> 189 us against 16-byte pieces of
  // 16 rows per store)
  __syncthreads();
  int8_t* const s_s8 = s_qx;
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const int p = 16 * pt + l16;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int nt = NTW * w + j;
      const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kHP + p) * NS + 16 * nt + 4 * lg;
      if (TAPS && a.tap_s32) *(int4*)(a.tap_s32 + so) = make_int4(acc[j][pt][0], acc[j][pt][1], acc[j][pt][2], acc[j][pt][3]);
      const uint32_t s8 = q8x4((float)acc[j][pt][0] * mreq[pt], (float)acc[j][pt][1] * mreq[pt],
                               (float)acc[j][pt][2] * mreq[pt], (float)acc[j][pt][3] * mreq[pt]);
      *(uint32_t*)&s_s8[p * NS + 16 * nt + 4 * lg] = s8;
      if (TAPS && a.tap_s8) *(uint32_t*)(a.tap_s8 + so) = s8;
    }
  }
  __syncthreads();
  static_assert(kHP * NS % (16 * kCT) == 0, "whole 16-byte pieces per thread");
  int8_t* const st8 = a.states + ((b * d.c + k) * H + h) * (int64_t)kHP * NS;
#pragma unroll
  for (int v = 0; v < kHP * NS / (16 * kCT); ++v)
    *(v4i*)(st8 + 16 * (tid + kCT * v)) = *(const v4i*)&s_s8[16 * (tid + kCT * v)];
}

// ===========================================================================
// k_cscan_i8: Y of one (batch, chunk, head). Four waves; wave w owns the row
// tiles {w, 7 - w, 8 + w, 15 - w} (l = 256) or {w, 7 - w} (l = 128), which
// balances the causal work. The x tile, the per-position tables and the passed
// state of chunk k - 1 are staged in LDS; the CB' fragments and Q(C) rows come
// from memory straight into registers.
// ===========================================================================
template <int DT, int LC, int NS>
__global__ __launch_bounds__(kCT, 3) void k_cscan_i8(ChunkArgs a) {
  typedef typename Store<DT>::T T;
  typedef FragF<DT> F;
  constexpr int RT = LC / 16, KN = NS / 64, NF = cb_frags(LC);
  constexpr int NTL = RT / 4;       // row tiles per wave
  constexpr int NU = LC * 8 / kCT;  // 16-byte x items per thread
  __shared__ __attribute__((aligned(16))) u16 s_x[LC * kHP];
  __shared__ __attribute__((aligned(16))) int8_t s_h8[kHP * NS];
  __shared__ __attribute__((aligned(16))) float s_va[LC];
  __shared__ __attribute__((aligned(16))) float s_vb[LC];
  __shared__ __attribute__((aligned(16))) float s_vw[4 * LC];
  const Dims& d = a.d;
  const BKH u = chunk_block(d, a.xcd_map);
  const int64_t b = u.b;
  const int k = u.k, h = u.h, H = d.H;
  const int g = h / d.hpg;
  const int tid = threadIdx.x;
  const int w = wave_id();
  const int lane = tid & (kWave - 1);
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)k * LC;
  const int64_t bh = b * H + h;
  const int64_t Lp = (int64_t)d.c * LC;
  const float scb = a.sc.s_C[g] * a.sc.s_B[g];
  const float Eg = (float)cb_exp(scb, NS);
  const float sC = a.sc.s_C[g];
  const float Dh = a.D[h];
  // the state steps of this lane's p values (16 pt + 4 lg + r), loaded first
  float4 ssr[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) ssr[pt] = ld_scale4(&a.sc.s_S[h * kHP + 16 * pt + 4 * lg]);
  // the passed state H_{k-1}: chunk k - 1's slot, the initial state, or none
  const int8_t* hprev = k > 0 ? a.states + ((b * d.c + k - 1) * H + h) * (int64_t)kHP * NS
                              : (a.init ? a.init + bh * (int64_t)kHP * NS : nullptr);

  // ---- staging ----
  {
    const int c8 = tid & 7, r0 = tid >> 3;
    const int64_t lim = d.L - 1 - t0;
    const int64_t rowB = (int64_t)H * kHP * sizeof(T);
    const char* xh = (const char*)a.X + ((b * d.L + t0) * H + h) * (int64_t)kHP * sizeof(T) + 16 * c8;
    v4i xr[NU];
#pragma unroll
    for (int v = 0; v < NU; ++v) xr[v] = __builtin_nontemporal_load((const v4i*)(xh + min((int64_t)(r0 + 32 * v), lim) * rowB));
    v4i hr[2];
    if (hprev) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int c = tid + kCT * v;  // 16-byte chunk of the state, < P N / 16
        if (c < kHP * NS / 16) hr[v] = *(const v4i*)(hprev + 16 * c);
      }
    }
    float va = 0.f, vd = 0.f;
    if (tid < LC) {
      va = a.dAcs[(bh * d.c + k) * (int64_t)LC + tid];
      const int64_t tv = t0 + min((int64_t)tid, lim);
      vd = Store<DT>::to_f(((const T*)a.dt)[(b * d.L + tv) * H + h]);
      if (t0 + tid >= d.L) vd = 0.f;
    }
#pragma unroll
    for (int v = 0; v < NU; ++v) *(v4i*)&s_x[xsw_off(r0 + 32 * v, 8 * c8)] = xr[v];
    if (hprev) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int c = tid + kCT * v;
        if (c < kHP * NS / 16) *(v4i*)&s_h8[bsw<NS>(c / (NS / 16), 16 * (c % (NS / 16)))] = hr[v];
      }
    }
    if (tid < LC) {
      float A2, B2;
      scan_vectors(va, vd, Eg, A2, B2);
      s_va[tid] = A2;
      s_vb[kperm(tid)] = B2;
    }
  }
  __syncthreads();

  float* Vw = s_vw + w * LC;
  int xoff[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) xoff[pt] = xsw_off(4 * lg + (l16 >> 2), 16 * pt + 4 * (l16 & 3));
  const uint32_t lane16 = 16u * (uint32_t)lane;
  const char* const cbk = (const char*)a.cbf + (((b * d.c + k) * d.G + g) * (int64_t)NF) * 1024;
  const uint32_t qc_lane = (uint32_t)(l16 * d.G * NS + 16 * lg);
  T* const ytile0 = (T*)a.Y + ((b * d.L + t0) * H + h) * (int64_t)kHP;

  struct TileOps {
    v4i off[RT / 2];
    v4i diag;
    v4i qc[KN];
  };
  const auto load_ops = [&](int i, TileOps& t) {
    const char* src = cbk + cb_frag_base(i) * 1024;
    // (with three workgroups per CU, skipping the pairs past the diagonal is
    // faster than a fixed load count: measured)
#pragma unroll
    for (int m = 0; m < RT / 2; ++m)
      if (m < i / 2) t.off[m] = *(const v4i*)(src + m * 1024 + lane16);
    t.diag = *(const v4i*)(src + (i / 2) * 1024 + lane16);
    const int8_t* qs = a.qC + ((b * Lp + t0 + 16 * i) * d.G + g) * (int64_t)NS;
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) t.qc[kn] = *(const v4i*)(qs + (qc_lane + 64 * kn));
  };
  const auto xfrags = [&](int m, F(&xf)[4]) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const v4s_t lo = ldtr16(s_x + xoff[pt] + (32 * m) * kHP);
      const v4s_t hi = ldtr16(s_x + xoff[pt] + (32 * m + 16) * kHP);
      xf[pt].v = __builtin_bit_cast(decltype(xf[pt].v), v8s_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
  };
  // Y^T[p, s] of row tile i (as in the head-persistent kernel)
  const auto scan_tile = [&](const int i, const TileOps& t) {
    const int mi = i >> 1;
    const int s_row = 16 * i + l16;
    const float a_ref = s_va[16 * i];
    for (int qq = lane; qq < 32 * mi; qq += kWave) Vw[qq] = __builtin_amdgcn_exp2f(a_ref - s_vb[qq]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    v4f acc[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] = v4f{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < RT / 2; ++m) {
      if (m < mi) {
        F xf[4];
        xfrags(m, xf);
        const float4 v0 = *(const float4*)&Vw[32 * m + 8 * lg];
        const float4 v1 = *(const float4*)&Vw[32 * m + 8 * lg + 4];
        const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        F wf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t dw = (uint32_t)t.off[m][e >> 1];
          const _Float16 c16 = __builtin_bit_cast(_Float16, (u16)((e & 1) ? (dw >> 16) : (dw & 0xffffu)));
          wf.set(e, __builtin_fmaf((float)c16, vv[e], 0.0f));
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = F::mma(xf[pt], wf, acc[pt]);
      }
    }
    const float a_s = s_va[s_row];
    const float us = __builtin_amdgcn_exp2f(a_s - a_ref);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[pt] *= us;
    if (hprev) {
      const float eo = __builtin_amdgcn_exp2f(a_s) * sC;
      v4i acc1[4];
#pragma unroll
      for (int kn = 0; kn < KN; ++kn) {
        v4i hb[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) hb[pt] = *(const v4i*)&s_h8[bsw<NS>(16 * pt + l16, 64 * kn + 16 * lg)];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc1[pt] = mma_i8(hb[pt], t.qc[kn], kn == 0 ? v4i{0, 0, 0, 0} : acc1[pt]);
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const float4 ss = ssr[pt];
        acc[pt][0] = fmaf((float)acc1[pt][0], eo * ss.x, acc[pt][0]);
        acc[pt][1] = fmaf((float)acc1[pt][1], eo * ss.y, acc[pt][1]);
        acc[pt][2] = fmaf((float)acc1[pt][2], eo * ss.z, acc[pt][2]);
        acc[pt][3] = fmaf((float)acc1[pt][3], eo * ss.w, acc[pt][3]);
      }
    }
    {
      F xd[4];
      xfrags(mi, xd);
      const float4 b0 = *(const float4*)&s_vb[32 * mi + 8 * lg];
      const float4 b1 = *(const float4*)&s_vb[32 * mi + 8 * lg + 4];
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      F wf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sp = 32 * mi + 16 * (e >> 2) + 4 * lg + (e & 3);
        const float arg = (sp <= s_row) ? a_s - bv[e] : -__builtin_inff();
        const float ev = __builtin_amdgcn_exp2f(arg);
        const uint32_t dw = (uint32_t)t.diag[e >> 1];
        const _Float16 c16 = __builtin_bit_cast(_Float16, (u16)((e & 1) ? (dw >> 16) : (dw & 0xffffu)));
        wf.set(e, __builtin_fmaf((float)c16, ev, (sp == s_row) ? Dh : 0.0f));
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) acc[pt] = F::mma(xd[pt], wf, acc[pt]);
    }
    // lanes of rows lg and lg ^ 1 (same l16) swap halves so that each lane
    // holds whole 16-byte pieces (8 consecutive p) and the row leaves in two
    // stores instead of four. Measured on the 64K-token layer: 549 us with
    // 8-byte pieces, 478 with the rows gathered through LDS, 468 this way.
    uint32_t dv[4][2];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      dv[pt][0] = pack2<DT>(acc[pt][0], acc[pt][1]);
      dv[pt][1] = pack2<DT>(acc[pt][2], acc[pt][3]);
    }
    const uint32_t om = (lg & 1) ? 0xffffffffu : 0u;  // bitwise selects (no indexed register arrays)
    uint32_t rv[2][2], kv[2][2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t v = (dv[q][e] & om) | (dv[2 + q][e] & ~om);  // odd rows send p tile q, even ones 2 + q
        kv[q][e] = (dv[2 + q][e] & om) | (dv[q][e] & ~om);          // and keep the other
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        rv[q][e] = (r[0] & om) | (r[1] & ~om);
      }
    if (t0 + s_row < d.L) {
      char* yrow = (char*)(ytile0 + (16 * i + l16) * (int64_t)H * kHP) + 8 * (lg & 2);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int jp = (lg & 1) ? 2 + q : q;
        // the lower 8 bytes come from the even row, the upper from the odd one
        const uint32_t l0 = (rv[q][0] & om) | (kv[q][0] & ~om), l1 = (rv[q][1] & om) | (kv[q][1] & ~om);
        const uint32_t h0 = (kv[q][0] & om) | (rv[q][0] & ~om), h1 = (kv[q][1] & om) | (rv[q][1] & ~om);
        *(v4i*)(yrow + 32 * jp) = v4i{(int)l0, (int)l1, (int)h0, (int)h1};
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // row tiles of this wave: w, 7 - w (, 8 + w, 15 - w); the next tile's
  // operands are issued before the current tile is scanned
  TileOps ta, tb;
  const auto tile_of = [&](int j) { return (j & 1) ? (8 * ((j >> 1) + 1) - 1 - w) : (8 * (j >> 1) + w); };
  load_ops(tile_of(0), ta);
#pragma unroll
  for (int j = 0; j < NTL; ++j) {
    if (j & 1) {
      if (j + 1 < NTL) load_ops(tile_of(j + 1), ta);
      scan_tile(tile_of(j), tb);
    } else {
      if (j + 1 < NTL) load_ops(tile_of(j + 1), tb);
      scan_tile(tile_of(j), ta);
    }
  }
}

}  // namespace

size_t chunked_i8_states_bytes(const Dims& d) { return (size_t)d.B * d.c * d.H * d.P * d.N; }

hipError_t launch_chunked_i8(const Dims& d, int dtype, const void* X, const void* dt, const int8_t* qC,
                             const int8_t* qbt, const u16* cbf, const float* dAcs, const float* lut,
                             const uint8_t* qdecay, const float* D, const ScalePtrs& sc, void* Y, const void* init,
                             void* final_state, int8_t* states, int8_t* tap_qxs, int32_t* tap_s32, int8_t* tap_s8,
                             int8_t* tap_passed, hipStream_t st) {
  const ChunkArgs ca{d, X, dt, qC, qbt, cbf, dAcs, lut, D, sc, states, (const int8_t*)init, Y, tap_qxs, tap_s32,
                     tap_s8, (int)((d.B * d.c * d.G) % 8 == 0)};
  const int64_t nb = d.B * (int64_t)d.c * d.H;
  if (nb == 0) return hipSuccess;
  if (nb >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const bool taps = tap_qxs || tap_s32 || tap_s8;
#define SSD_CS(DTV, LCV, NSV)                                                                              \
  if (dtype == DTV && d.l == LCV && d.N == NSV) {                                                          \
    if (taps)                                                                                              \
      hipLaunchKernelGGL((k_cstate_i8<DTV, LCV, NSV, true>), dim3((unsigned)nb), dim3(kCT), 0, st, ca);  \
    else                                                                                                   \
      hipLaunchKernelGGL((k_cstate_i8<DTV, LCV, NSV, false>), dim3((unsigned)nb), dim3(kCT), 0, st, ca); \
    e = hipGetLastError();                                                                                 \
  }
  hipError_t e = hipErrorNotSupported;
  SSD_CS(DT_F16, 256, 128)
  SSD_CS(DT_F16, 256, 64)
  SSD_CS(DT_F16, 128, 128)
  SSD_CS(DT_F16, 128, 64)
  SSD_CS(DT_BF16, 256, 128)
  SSD_CS(DT_BF16, 256, 64)
  SSD_CS(DT_BF16, 128, 128)
  SSD_CS(DT_BF16, 128, 64)
#undef SSD_CS
  if (e != hipSuccess) return e;
  e = launch_state_passing(d, true, states, nullptr, qdecay, init, final_state, st);
  if (e != hipSuccess) return e;
  if (tap_passed) {
    e = hipMemcpyAsync(tap_passed, states, chunked_i8_states_bytes(d), hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
  }
  e = hipErrorNotSupported;
#define SSD_SC(DTV, LCV, NSV)                                                                           \
  if (dtype == DTV && d.l == LCV && d.N == NSV) {                                                       \
    hipLaunchKernelGGL((k_cscan_i8<DTV, LCV, NSV>), dim3((unsigned)nb), dim3(kCT), 0, st, ca);         \
    e = hipGetLastError();                                                                              \
  }
  SSD_SC(DT_F16, 256, 128)
  SSD_SC(DT_F16, 256, 64)
  SSD_SC(DT_F16, 128, 128)
  SSD_SC(DT_F16, 128, 64)
  SSD_SC(DT_BF16, 256, 128)
  SSD_SC(DT_BF16, 256, 64)
  SSD_SC(DT_BF16, 128, 128)
  SSD_SC(DT_BF16, 128, 64)
#undef SSD_SC
  return e;
}

}  // namespace ssd
