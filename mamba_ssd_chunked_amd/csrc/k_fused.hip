// Fused SSD forward on the float path (fp16 or bf16 inputs): ChunkCumsum, then
// one workgroup of eight waves per (batch, head) walking that head's chunks in
// order with the fp32 state in registers. The fused INT8 path is in
// k_fused_i8.hip.
//
// ChunkScan2 factorisation (exact algebra): for a column tile j strictly below
// row tile i, exp(a_s - a_s') = u_s * V_i[s'] with u_s = exp(a_s - a_{16i}) <= 1
// and V_i[s'] = exp(a_{16i} - a_s') <= 1, so each row tile needs one table V_i
// and one factor per output row instead of an exponential per element.
// Off-diagonal tiles accumulate unscaled and are multiplied by u_s once; the
// diagonal tile uses exp(a_s - a_s') directly.
#include "ssd_cumsum.hpp"
#include "ssd_device.hpp"
#include "ssd_fused.hpp"
#include "ssd_launch.hpp"

namespace ssd {
namespace {

constexpr int kP = 64;        // head dim of the fused kernel
constexpr int kThreads = 512;  // eight waves
constexpr int kWaves = kThreads / kWave;
constexpr float kLog2e = 1.4426950408889634f;

// 2^x with the hardware transcendental (arguments here are <= 0; results that
// would be denormal flush to 0, far below anything that reaches the output).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS layouts. Rows are split into 16-byte chunks whose index is XOR-swizzled
// with low row bits, so the 8 or 16 lanes served together hit distinct banks.
// ---------------------------------------------------------------------------
// x transposed, [p][s'] in 2-byte elements, with s reordered inside each block
// of 32 positions (two 16-position column tiles 2m and 2m + 1): the 4-position
// runs s = 32m + 16h + 4g + (0..3) sit at 32m + 8g + 4h + (0..3). A lane's
// ChunkScan2 operand (group g of tiles 2m and 2m + 1) is then one 16-byte
// chunk, index 4m + g. Rows of LC elements; the chunk index is XORed with the
// row's low four bits and, in bit 2, with row bit 4 (as the (LUT x)^T tile), so
// the operand reads (16 consecutive rows, one chunk) and each half wave of the
// staging writes land on distinct bank positions. (Rows padded by 16 bytes
// instead of XORed, an earlier layout, left the operand reads with bank
// conflicts: about half of the kernel's remaining ones, measured by a probe.)
template <int LC>
__device__ __forceinline__ int xT_pair(int p, int m, int g) {  // 16-byte chunk start
  return p * LC + 8 * ((4 * m + g) ^ (p & 15) ^ (((p >> 4) & 1) << 2));
}
// byte tiles [rows][W]; c a byte column aligned to 4
template <int W>
__device__ __forceinline__ int b_off(int r, int c) {
  constexpr int nch = W / 16;
  return r * W + 16 * ((c >> 4) ^ (r & (nch - 1) & 7)) + (c & 15);
}

// Eight 2-byte input values read from LDS as an MFMA operand fragment.
template <int DT>
__device__ __forceinline__ FragF<DT> frag16(const u16* p) {
  FragF<DT> f;
  if constexpr (DT == DT_F16)
    f.v = *(const v8h*)p;
  else
    f.v = *(const v8bf*)p;
  return f;
}

// ===========================================================================
// Fused float forward (fp16 or bf16 inputs). The same per-head walk over the
// chunks as the INT8 kernel, with every contraction on MFMA in the input's
// 16-bit type (fp32 accumulation):
//   ChunkState   S^T[n,p] = sum_s B^T[n,s] (LUT x)^T[s,p]  (B^T by transposing
//                LDS reads of the B rows, LUT x rounded to the 16-bit type);
//   StatePassing H_k = exp(a_{k,l-1}) H_{k-1} + S_k, in fp32 registers;
//   ChunkScan1   Y_off = exp(a_s) sum_n C[s,n] H_{k-1}[p,n] (H as 16-bit in LDS);
//   ChunkBMM/Scan2 as in the INT8 kernel, CB from the B and C rows.
// bf16 keeps 8 significant bits, so with bf16 inputs the computed operands (LUT
// B in ChunkState, the Scan2 weights and the state copy ChunkScan1 reads) are
// carried as hi + lo pairs (two MFMAs, about 16 significant bits); B, C and x
// are exact inputs.
// ===========================================================================

// fp16 tiles [rows][W] (element offsets); 16-byte chunks XOR-swizzled with the
// low row bits (up to 16 distinct chunks for the 16 lanes read together)
template <int W>
__device__ __forceinline__ int h_off(int r, int c) {
  constexpr int nch = W / 8;
  constexpr int msk = (nch < 16 ? nch : 16) - 1;
  return r * W + 8 * ((c >> 3) ^ (r & msk)) + (c & 7);
}

// The 16-bit (LUT x)^T tile [p][s] (element offsets): h_off's row XOR, and row
// bit 4 also XORed into bit 2 of the chunk index. The staging writes one column
// chunk of rows 8 c8 + e (c8 = 0..7) per instruction; with the low row bits
// alone, rows 16 apart shared a chunk (four-way bank conflicts, the kernel's
// largest source of them); now they spread over all 16 positions. The
// ChunkState reads (16 consecutive rows, bit 4 fixed) stay on 16 distinct
// chunks.
template <int W>
__device__ __forceinline__ int xs_off(int r, int c) {
  constexpr int nch = W / 8;
  constexpr int msk = (nch < 16 ? nch : 16) - 1;
  static_assert(nch >= 8, "room for chunk bit 2");
  return r * W + 8 * ((c >> 3) ^ (r & msk) ^ (((r >> 4) & 1) << 2)) + (c & 7);
}
typedef short v4s __attribute__((ext_vector_type(4)));
// Transposing LDS read (16-bit elements): the 16 lanes of a group each point at
// 8 bytes; lanes 4r .. 4r + 3 form row r (16 elements) of a 4 x 16 matrix, and
// lane i receives column i (element i of rows 0..3).
__device__ __forceinline__ v4s lds_tr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(u16*)p);
}

typedef short v8s __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v8s v8s_join(v4s lo, v4s hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int DT>
__device__ __forceinline__ FragF<DT> frag_u4(const uint4& v) {
  FragF<DT> f;
  f.v = __builtin_bit_cast(decltype(f.v), v);
  return f;
}

// 16-bit storage bits of a float, and its rounding residual (for hi + lo pairs)
template <int DT>
__device__ __forceinline__ uint32_t bits16(float v) {
  return (uint32_t)__builtin_bit_cast(u16, Store<DT>::from_f(v));
}
template <int DT>
__device__ __forceinline__ float resid16(float v) {
  return v - Store<DT>::to_f(Store<DT>::from_f(v));
}

struct FusedFArgs {
  Dims d;
  const void* X;
  const void* dt;
  const void* B;
  const void* C;
  const float* dAcs;
  const float* lut;
  const float* D;
  void* Y;
  const float* init;  // optional initial state [B,H,P,N] fp32
  float* final_state;
  int64_t nfull;  // blocks [0, nfull) run whole heads, the rest p halves (block_head)
  int unit_map;
  int half_il;
};

// LDS arrays of the float kernel, declared once per kernel (see k_fused_i8)
template <int DT, int LC, int NS>
struct FLds {
  static constexpr bool SPLIT = DT == DT_BF16;
  u16* xT;    // x^T (xT_pair layout)
  u16* xs;    // 16-bit (LUT x)^T [p][s] (xs_off<LC>); with bf16 the LUT goes on the B side
  u16* B;     // B rows [s][n] (h_off<NS>)
  u16* H;     // 16-bit passed state [p][n] (h_off<NS>)
  u16* H_lo;  // its residual (bf16)
  float* vec; // a*log2(e), dt (, LUT)
  float* vw;
};

// PW = 4: a whole head per workgroup; PW = 2: p tiles 2 ph, 2 ph + 1 of a head
// (the partial last round, as in the INT8 kernel).
template <int DT, int LC, int NS, int PW>
__device__ __forceinline__ void fused_f16_body(const FusedFArgs& a, const int64_t bx, const FLds<DT, LC, NS>& ls) {
  typedef typename Store<DT>::T T;
  typedef FragF<DT> F;
  constexpr bool SPLIT = DT == DT_BF16;  // hi + lo pairs for LUT x and the weights
  constexpr int RT = LC / 16;            // row tiles of the chunk
  constexpr int NT = NS / 16;            // n tiles of the state
  constexpr int PTW = PW * NT / kWaves;  // p tiles per wave in ChunkState / StatePassing
  constexpr int KSF = LC / 32;           // ChunkState K steps (fp16 MFMA, K = 32)
  constexpr int KNF = NS / 32;           // K steps over N
  constexpr int C8N = 2 * PW;            // 8-column groups of p staged by this workgroup
  constexpr int XI = (LC / 4) * C8N;     // staging items (4 rows x 8 p each)
  static_assert(XI <= kThreads, "tile split");

  u16* const s_xT = ls.xT;
  u16* const s_xs = ls.xs;
  u16* const s_B = ls.B;
  u16* const s_H = ls.H;
  u16* const s_H_lo = ls.H_lo;
  float* const s_vec = ls.vec;
  float* const s_vw = ls.vw;
  const float* vA2 = s_vec;
  const float* vDt = s_vec + LC;
  const float* vLut = s_vec + 2 * LC;  // bf16 only

  const Dims& d = a.d;
  // bx: the block's index within its part of the launch
  const BlockHead bh = block_head<PW>(d, bx, a.nfull, a.unit_map, a.half_il);
  const int64_t unit = bh.unit, hl = bh.hl;
  const int ph = bh.ph;
  const int pt_base = (PW == 4) ? 0 : 2 * ph;
  const int c8b = 2 * pt_base;  // first 8-column group of p
  const int64_t b = unit / d.G;
  const int g_h = (int)(unit % d.G);
  const int h = g_h * d.hpg + (int)hl;
  const int w = wave_id();
  const int H = d.H;
  const int nt_own = w % NT;
  const int pt0 = pt_base + (w / NT) * PTW;
  const float Dh = a.D[h];
  const int tid0 = threadIdx.x;
  float* Vw = s_vw + w * LC;
  T* const ybase = (T*)a.Y + (b * d.L * H + h) * (int64_t)kP;
  const T* const Xb = (const T*)a.X + (b * d.L * H + h) * (int64_t)kP;
  const T* const Bb = (const T*)a.B + (b * d.L * d.G + g_h) * (int64_t)NS;
  const T* const Cb = (const T*)a.C + (b * d.L * d.G + g_h) * (int64_t)NS;
  const int rowB = d.G * NS;  // elements between consecutive positions of B / C
  const int rowX = H * kP;    // elements between consecutive positions of x

  // staging of chunk kc: x^T, fp16(LUT x)^T and the per-position vectors
  struct Pf {
    uint4 x[4];
    float4 lut;
    float va;
    float vl;  // LUT of position tid % LC (bf16 only)
    uint32_t vd;
  };
  // staging item it -> rows 4q .. 4q + 3, columns 8 c8 .. 8 c8 + 7 of the chunk.
  // For whole heads the lane bits are dealt out so that every half wave's LDS
  // writes (x^T and (LUT x)^T) land on 32 distinct 8-byte bank positions: lane
  // bits 0-1 and 5 are c8's bits 0-1 and 2, bit 2 is q's bit 2 (the 8-byte
  // half of an x^T chunk), bits 3-4 are q's bits 0-1; before, the half was
  // lane bit 5 and each half wave wrote one half of 16 chunks (two-way bank
  // conflicts). The wave index gives q's higher bits.
  const auto stage_item = [&](int it, int& q, int& c8) {
    if constexpr (C8N == 8) {
      const int ln = it & (kWave - 1);
      c8 = (ln & 3) | (((ln >> 5) & 1) << 2);
      q = 8 * (it >> 6) + (((ln >> 2) & 1) << 2) + ((ln >> 3) & 3);
    } else {
      q = it / C8N;
      c8 = c8b + it % C8N;
    }
  };
  const auto stage_load = [&](int kc, int tid, Pf& pf) {
    const int t0 = kc * LC;
    const int lim = min(LC - 1, (int)d.L - 1 - t0);
    const int it = tid % XI;
    int q, c8;
    stage_item(it, q, c8);
    const T* xk = Xb + (int64_t)t0 * rowX + 8 * c8;
#pragma unroll
    for (int r = 0; r < 4; ++r) pf.x[r] = *(const uint4*)(xk + __umul24(min(4 * q + r, lim), rowX));
    const int64_t cs0 = ((b * H + h) * d.c + kc) * (int64_t)LC;
    pf.lut = *(const float4*)(a.lut + cs0 + 4 * q);
    const int sv = tid % LC;
    pf.va = a.dAcs[cs0 + sv];
    if constexpr (SPLIT) pf.vl = a.lut[cs0 + sv];
    pf.vd = ((const u16*)a.dt)[((b * d.L + t0) * H + h) + __umul24(min(sv, lim), H)];
  };
  const auto stage_store = [&](int kc, int tid, const Pf& pf) {
    const int t0 = kc * LC;
    // every prefetched register passes through an empty asm in all lanes (see
    // prefetch_store of the INT8 kernel)
    uint4 xr[4] = {pf.x[0], pf.x[1], pf.x[2], pf.x[3]};
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(xr[r].x), "+v"(xr[r].y), "+v"(xr[r].z), "+v"(xr[r].w));
    float4 lutp = pf.lut;
    float vap = pf.va, vlp = SPLIT ? pf.vl : 0.f;
    uint32_t vdp = pf.vd;
    asm volatile("" : "+v"(lutp.x), "+v"(lutp.y), "+v"(lutp.z), "+v"(lutp.w), "+v"(vap), "+v"(vdp));
    if constexpr (SPLIT) asm volatile("" : "+v"(vlp));
    if (tid < XI) {
      int q, c8;
      stage_item(tid, q, c8);
      const uint32_t* w0 = (const uint32_t*)&xr[0];
      const uint32_t* w1 = (const uint32_t*)&xr[1];
      const uint32_t* w2 = (const uint32_t*)&xr[2];
      const uint32_t* w3 = (const uint32_t*)&xr[3];
      const int hx = 4 * ((q >> 2) & 1);  // the 8-byte half of the chunk (h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *(uint2*)(s_xT + xT_pair<LC>(8 * c8 + 2 * e, q >> 3, q & 3) + hx) =
            make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u), __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u));
        *(uint2*)(s_xT + xT_pair<LC>(8 * c8 + 2 * e + 1, q >> 3, q & 3) + hx) =
            make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u), __builtin_amdgcn_perm(w3[e], w2[e], 0x07060302u));
      }
      // fl32(LUT x) in the 16-bit type for 4 rows of each p (fp16 only)
      if constexpr (!SPLIT) {
        const float lutv[4] = {lutp.x, lutp.y, lutp.z, lutp.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t dw = (e >> 1) == 0 ? xr[r].x : (e >> 1) == 1 ? xr[r].y : (e >> 1) == 2 ? xr[r].z : xr[r].w;
            const uint32_t hv = (e & 1) ? (dw >> 16) : (dw & 0xffffu);
            v[r] = __builtin_fmaf(lutv[r], Store<DT>::to_f(__builtin_bit_cast(T, (u16)hv)), 0.0f);
          }
          *(uint2*)&s_xs[xs_off<LC>(8 * c8 + e, 4 * q)] = make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
        }
      }
    }
    if (tid < LC) {
      s_vec[tid] = vap * kLog2e;
      const float dtv = Store<DT>::to_f(__builtin_bit_cast(T, (u16)vdp));
      s_vec[LC + tid] = (t0 + tid < (int)d.L) ? dtv : 0.f;
      if constexpr (SPLIT) s_vec[2 * LC + tid] = vlp;
    }
  };
  // B rows of chunk kc straight into LDS (1 KB per copy; lane L fills bytes
  // 16 L .. 16 L + 15, its source chosen to give the h_off<NS> layout)
  const auto dma_B = [&](int kc, int lane) {
    constexpr int OPS = LC * NS * 2 / 1024;
    constexpr int msk = (NS / 8 < 16 ? NS / 8 : 16) - 1;
    const int t0 = kc * LC;
    const int lim = min(LC - 1, (int)d.L - 1 - t0);
    const T* src0 = Bb + (int64_t)t0 * rowB;
#pragma unroll
    for (int gi = w; gi < OPS; gi += kWaves) {
      const int byte = 1024 * gi + 16 * lane;
      const int r = byte / (2 * NS), pc = (byte % (2 * NS)) / 16;
      const int c = pc ^ (r & msk);
      __builtin_amdgcn_global_load_lds((const void*)(src0 + (__umul24(min(r, lim), rowB) + 8 * c)),
                                       (__attribute__((address_space(3))) void*)((char*)s_B + 1024 * gi), 16, 0, 0);
    }
  };
  // the wave index, hidden from the compiler at every chunk of the main loop so
  // that what derives from it is formed per chunk rather than hoisted and
  // spilled
  int wk = w;
  // C rows (B operand over N) of this wave's row tiles {w, 15 - w}
  // C rows of row tile {w, 15 - w}[rr] of chunk kc
  const auto load_C = [&](int kc, int lane, int rr, uint4 (&cf)[KNF]) {
    const int t0 = kc * LC;
    const int lim = min(LC - 1, (int)d.L - 1 - t0);
    const int l16 = lane & 15, lg = lane >> 4;
    const T* c0 = Cb + (int64_t)t0 * rowB;
    const int i = min((rr == 0) ? wk : 2 * kWaves - 1 - wk, RT - 1);
    const T* src = c0 + (__umul24(min(16 * i + l16, lim), rowB) + 8 * lg);
#pragma unroll
    for (int kn = 0; kn < KNF; ++kn) cf[kn] = *(const uint4*)(src + 32 * kn);
  };

  float Hs[PTW][4];  // fp32 state: lane (p = 16 (pt0 + j) + lane % 16, n = 16 nt_own + 4 (lane / 16) + r)
  const bool has_init = a.init != nullptr;
  {
    const int l16 = tid0 & 15, lg = (tid0 & (kWave - 1)) >> 4;
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int p = 16 * (pt0 + j) + l16;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (has_init) v = *(const float4*)(a.init + ((b * H + h) * (int64_t)kP + p) * NS + 16 * nt_own + 4 * lg);
      Hs[j][0] = v.x;
      Hs[j][1] = v.y;
      Hs[j][2] = v.z;
      Hs[j][3] = v.w;
      if (has_init) {  // 16-bit copy (bf16: hi + lo) for chunk 0's ChunkScan1
        const int ho = h_off<NS>(p, 16 * nt_own + 4 * lg);
        *(uint2*)&s_H[ho] =
            make_uint2(bits16<DT>(v.x) | (bits16<DT>(v.y) << 16), bits16<DT>(v.z) | (bits16<DT>(v.w) << 16));
        if constexpr (SPLIT)
          *(uint2*)&s_H_lo[ho] = make_uint2(bits16<DT>(resid16<DT>(v.x)) | (bits16<DT>(resid16<DT>(v.y)) << 16),
                                            bits16<DT>(resid16<DT>(v.z)) | (bits16<DT>(resid16<DT>(v.w)) << 16));
      }
    }
  }

  uint4 cf2[2][KNF];
  {  // chunk 0
    Pf pf;
    dma_B(0, tid0 & (kWave - 1));
    load_C(0, tid0 & (kWave - 1), 0, cf2[0]);
    load_C(0, tid0 & (kWave - 1), 1, cf2[1]);
    stage_load(0, tid0, pf);
    stage_store(0, tid0, pf);
  }

  for (int k = 0; k < d.c; ++k) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int l16 = lane & 15, lg = lane >> 4;
    const int64_t t0 = (int64_t)k * LC;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // B rows and C rows have landed
    __syncthreads();  // chunk k staged; s_H holds H_{k-1}
    asm volatile("" : "+s"(wk));
    // issue priority: the second wave of each SIMD (w + 4) leads ChunkState
    // and the first row tile, the first wave the second tile, so that neither
    // falls behind and runs alone at the end of the chunk (as in the INT8
    // kernel; measured 2% faster here)
    if (wk >= 4) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
    const float alast2 = vA2[LC - 1];  // a_{k,l-1} log2(e): StatePassing decay

#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int kn = 0; kn < KNF; ++kn)
        asm volatile("" : "+v"(cf2[rr][kn].x), "+v"(cf2[rr][kn].y), "+v"(cf2[rr][kn].z), "+v"(cf2[rr][kn].w));
    const int kn1 = min(k + 1, d.c - 1);
    Pf pf;
    stage_load(kn1, tid, pf);  // issued before ChunkState (as in the INT8 kernel)
    // the next chunk's C rows of row tile 15 - w now, those of tile w once the
    // scan is done with them (as in the INT8 kernel)
    uint4 cfn1[KNF];
    load_C(kn1, lane, 1, cfn1);

    // ---- ChunkState^T for (n tile nt_own, p tiles pt0 ..) ----
    v4f sacc[PTW];
    const int cn = 16 * nt_own + 4 * (l16 & 3);
    if constexpr (!SPLIT) {
      // A: B^T rows n = 16 nt_own + l16, K = s0 .. s0 + 7 (two reads of 4 rows);
      // the operands of step ks + 1 are read while step ks multiplies
      F fa[2], fb[2][PTW];
      const auto load_ks = [&](int ks, F& a_, F (&b_)[PTW]) {
        const int s0 = 32 * ks + 8 * lg;
        const v4s lo = lds_tr16(s_B + h_off<NS>(s0 + (l16 >> 2), cn));
        const v4s hi = lds_tr16(s_B + h_off<NS>(s0 + 4 + (l16 >> 2), cn));
        a_.v = __builtin_bit_cast(decltype(a_.v), v8s_join(lo, hi));
#pragma unroll
        for (int j = 0; j < PTW; ++j) b_[j] = frag16<DT>(&s_xs[xs_off<LC>(16 * (pt0 + j) + l16, s0)]);
      };
      load_ks(0, fa[0], fb[0]);
#pragma unroll
      for (int ks = 0; ks < KSF; ++ks) {
        if (ks + 1 < KSF) load_ks(ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
#pragma unroll
        for (int j = 0; j < PTW; ++j)
          sacc[j] = F::mma(fa[ks & 1], fb[ks & 1][j], ks == 0 ? v4f{0, 0, 0, 0} : sacc[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PTW; ++j) sacc[j] = v4f{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KSF; ++ks) {
        // bf16: S^T = (B LUT)^T x, with B LUT formed here as hi + lo and x read
        // exactly from x^T. K order of x^T's operand: s = 32 ks + 4 lg + (0..3)
        // and 32 ks + 16 + 4 lg + (0..3); the two transposing reads follow it.
        const int sA = 32 * ks + 4 * lg, sB = sA + 16;
        const v4s lo = lds_tr16(s_B + h_off<NS>(sA + (l16 >> 2), cn));
        const v4s hi = lds_tr16(s_B + h_off<NS>(sB + (l16 >> 2), cn));
        const float4 la = *(const float4*)&vLut[sA];
        const float4 lb = *(const float4*)&vLut[sB];
        const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
        F fh, fl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const short bs = e < 4 ? lo[e] : hi[e - 4];
          const float v = Store<DT>::to_f(__builtin_bit_cast(T, (u16)bs)) * lv[e];
          fh.set(e, v);
          fl.set(e, resid16<DT>(v));
        }
#pragma unroll
        for (int j = 0; j < PTW; ++j) {
          const F fb = frag16<DT>(&s_xT[xT_pair<LC>(16 * (pt0 + j) + l16, ks, lg)]);
          sacc[j] = F::mma(fh, fb, sacc[j]);
          sacc[j] = F::mma(fl, fb, sacc[j]);
        }
      }
    }

    // ---- ChunkScan, transposed: Y^T[p, s] for row tiles {w, 15 - w} ----
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int i = (rr == 0) ? wk : 2 * kWaves - 1 - wk;
      if (rr == 1) { if (wk >= 4) __builtin_amdgcn_s_setprio(0); else __builtin_amdgcn_s_setprio(1); }
      if (i >= RT) continue;
      const int s_row = 16 * i + l16;
      F cr[KNF];
#pragma unroll
      for (int kn = 0; kn < KNF; ++kn) cr[kn] = frag_u4<DT>(rr ? cf2[1][kn] : cf2[0][kn]);
      // V_i[s'] = exp(a_{16i} - a_s') dt_s' for s' < 16 i
      const float a_ref = vA2[16 * i];
      for (int sp = lane; sp < 16 * i; sp += kWave) Vw[sp] = fast_exp2(a_ref - vA2[sp]) * vDt[sp];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      v4f acc[PW];
      // off-diagonal pairs (jA, jA + 1); the first one starts the accumulators
      const auto pair = [&](int jA, bool first) {
        const int jB = jA + 1;
        v4f cbA = v4f{0, 0, 0, 0}, cbB = v4f{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < KNF; ++kn)
          cbA = F::mma(frag16<DT>(&s_B[h_off<NS>(16 * jA + l16, 32 * kn + 8 * lg)]), cr[kn], cbA);
#pragma unroll
        for (int kn = 0; kn < KNF; ++kn)
          cbB = F::mma(frag16<DT>(&s_B[h_off<NS>(16 * jB + l16, 32 * kn + 8 * lg)]), cr[kn], cbB);
        const float4 vA = *(const float4*)&Vw[16 * jA + 4 * lg];
        const float4 vB = *(const float4*)&Vw[16 * jB + 4 * lg];
        const float wv[8] = {cbA[0] * vA.x, cbA[1] * vA.y, cbA[2] * vA.z, cbA[3] * vA.w,
                             cbB[0] * vB.x, cbB[1] * vB.y, cbB[2] * vB.z, cbB[3] * vB.w};
        F wf, wl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          wf.set(e, wv[e]);
          if constexpr (SPLIT) wl.set(e, resid16<DT>(wv[e]));
        }
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) {
          const F xf = frag16<DT>(&s_xT[xT_pair<LC>(16 * (pt_base + jp) + l16, jA >> 1, lg)]);
          acc[jp] = F::mma(xf, wf, first ? v4f{0, 0, 0, 0} : acc[jp]);
          if constexpr (SPLIT) acc[jp] = F::mma(xf, wl, acc[jp]);
        }
      };
      if (i >= 2) {
        pair(0, true);
        for (int jA = 2; jA + 1 < i; jA += 2) pair(jA, false);
      } else {
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) acc[jp] = v4f{0, 0, 0, 0};
      }
      const float a_s = vA2[s_row];
      const float us = fast_exp2(a_s - a_ref);
#pragma unroll
      for (int jp = 0; jp < PW; ++jp) acc[jp] *= us;
      // ChunkScan1: exp(a_s) sum_n C[s,n] H_{k-1}[p,n] (H_{-1}: the initial state)
      // (the p tiles' MFMA chains interleave: each K step reads the operands of
      // all p tiles first)
      if (k > 0 || has_init) {
        const float eo = fast_exp2(a_s);
        v4f acc1[PW];
#pragma unroll
        for (int kn = 0; kn < KNF; ++kn) {
          F hf[PW], hl[PW];
#pragma unroll
          for (int jp = 0; jp < PW; ++jp) {
            const int ho = h_off<NS>(16 * (pt_base + jp) + l16, 32 * kn + 8 * lg);
            hf[jp] = frag16<DT>(&s_H[ho]);
            if constexpr (SPLIT) hl[jp] = frag16<DT>(&s_H_lo[ho]);
          }
#pragma unroll
          for (int jp = 0; jp < PW; ++jp) {
            acc1[jp] = F::mma(hf[jp], cr[kn], kn == 0 ? v4f{0, 0, 0, 0} : acc1[jp]);
            if constexpr (SPLIT) acc1[jp] = F::mma(hl[jp], cr[kn], acc1[jp]);
          }
        }
#pragma unroll
        for (int jp = 0; jp < PW; ++jp)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[jp][r] = fmaf(acc1[jp][r], eo, acc[jp][r]);
      }
      {  // diagonal tile (D on its diagonal), sharing its MFMA with tile i - 1 (odd i)
        const int hd = i & 1;
        const int jL = i - 1;
        v4f cbD = v4f{0, 0, 0, 0}, cbL = v4f{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < KNF; ++kn)
          cbD = F::mma(frag16<DT>(&s_B[h_off<NS>(16 * i + l16, 32 * kn + 8 * lg)]), cr[kn], cbD);
        if (hd) {
#pragma unroll
          for (int kn = 0; kn < KNF; ++kn)
            cbL = F::mma(frag16<DT>(&s_B[h_off<NS>(16 * jL + l16, 32 * kn + 8 * lg)]), cr[kn], cbL);
        }
        const float4 ad = *(const float4*)&vA2[16 * i + 4 * lg];
        const float4 dd = *(const float4*)&vDt[16 * i + 4 * lg];
        float4 vL = make_float4(0.f, 0.f, 0.f, 0.f);
        if (hd) vL = *(const float4*)&Vw[16 * jL + 4 * lg];
        const float adv[4] = {ad.x, ad.y, ad.z, ad.w};
        const float ddv[4] = {dd.x, dd.y, dd.z, dd.w};
        const float vLv[4] = {vL.x * us, vL.y * us, vL.z * us, vL.w * us};
        float wd[4], wl[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sp = 16 * i + 4 * lg + r;
          const float wv = cbD[r] * fast_exp2(a_s - adv[r]) * ddv[r];  // selected below (no branch)
          wd[r] = (sp < s_row) ? wv : (sp == s_row) ? wv + Dh : 0.f;
          wl[r] = cbL[r] * vLv[r];
        }
        F wf, wlo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v0 = hd ? wl[r] : wd[r], v1 = hd ? wd[r] : 0.f;
          wf.set(r, v0);
          wf.set(r + 4, v1);
          if constexpr (SPLIT) {
            wlo.set(r, resid16<DT>(v0));
            wlo.set(r + 4, resid16<DT>(v1));
          }
        }
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) {
          const F xf = frag16<DT>(&s_xT[xT_pair<LC>(16 * (pt_base + jp) + l16, i >> 1, lg)]);
          acc[jp] = F::mma(xf, wf, acc[jp]);
          if constexpr (SPLIT) acc[jp] = F::mma(xf, wlo, acc[jp]);
        }
      }
      const int64_t t = t0 + s_row;
      char* yrow = (char*)ybase + (__umul24((uint32_t)t, H * kP * 2) + 4 * lg * 2);
#pragma unroll
      for (int jp = 0; jp < PW; ++jp) {
        const int pt = pt_base + jp;
        if (t < d.L)
          *(uint2*)(yrow + 32 * pt) = make_uint2(pack2<DT>(acc[jp][0], acc[jp][1]), pack2<DT>(acc[jp][2], acc[jp][3]));
      }
      __builtin_amdgcn_wave_barrier();
      if (rr == 0) load_C(kn1, lane, 0, cf2[0]);
    }
    __syncthreads();  // chunk k's tiles and s_H are no longer read
    stage_store(kn1, tid, pf);
    dma_B(kn1, lane);

    // ---- StatePassing in fp32 registers; 16-bit copy for the next ChunkScan1 ----
    const float decay = fast_exp2(alast2);
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Hs[j][r] = (k == 0 && !has_init) ? sacc[j][r] : fmaf(decay, Hs[j][r], sacc[j][r]);
      const int p = 16 * (pt0 + j) + l16;
      const int ho = h_off<NS>(p, 16 * nt_own + 4 * lg);
      *(uint2*)&s_H[ho] = make_uint2(pack2<DT>(Hs[j][0], Hs[j][1]), pack2<DT>(Hs[j][2], Hs[j][3]));
      if constexpr (SPLIT)
        *(uint2*)&s_H_lo[ho] =
            make_uint2(pack2<DT>(resid16<DT>(Hs[j][0]), resid16<DT>(Hs[j][1])),
                       pack2<DT>(resid16<DT>(Hs[j][2]), resid16<DT>(Hs[j][3])));
    }
#pragma unroll
    for (int kn = 0; kn < KNF; ++kn) cf2[1][kn] = cfn1[kn];
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (a.final_state) {
    const int l16 = tid0 & 15, lg = (tid0 & (kWave - 1)) >> 4;
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int p = 16 * (pt0 + j) + l16;
      const int64_t fo = ((b * H + h) * (int64_t)kP + p) * NS + 16 * nt_own + 4 * lg;
      *(float4*)(a.final_state + fo) = make_float4(Hs[j][0], Hs[j][1], Hs[j][2], Hs[j][3]);
    }
  }
}

// whole heads and p halves in one launch (as k_fused_i8)
template <int DT, int LC, int NS>
__global__ __launch_bounds__(kThreads, 1) void k_fused_f16(FusedFArgs a) {
  constexpr bool SPLIT = DT == DT_BF16;
  __shared__ __attribute__((aligned(16))) u16 s_xT[kP * LC];
  __shared__ __attribute__((aligned(16))) u16 s_xs[SPLIT ? 8 : kP * LC];
  __shared__ __attribute__((aligned(16))) u16 s_B[LC * NS];
  __shared__ __attribute__((aligned(16))) u16 s_H[kP * NS];
  __shared__ __attribute__((aligned(16))) u16 s_H_lo[SPLIT ? kP * NS : 8];
  __shared__ __attribute__((aligned(16))) float s_vec[(SPLIT ? 3 : 2) * LC];
  __shared__ __attribute__((aligned(16))) float s_vw[kWaves * LC];
  const FLds<DT, LC, NS> ls{s_xT, s_xs, s_B, s_H, s_H_lo, s_vec, s_vw};
  const int64_t bid = blockIdx.x;
  if (bid < a.nfull)
    fused_f16_body<DT, LC, NS, 4>(a, bid, ls);
  else
    fused_f16_body<DT, LC, NS, 2>(a, bid - a.nfull, ls);
}

constexpr size_t kAl = 256;
size_t al(size_t v) { return (v + kAl - 1) / kAl * kAl; }

// One workgroup per CU at a time: B*H heads run in ceil(B*H / CUs) rounds. When
// the last round is at most half full, its heads are split in two p halves so
// the round spreads over all CUs (each half recomputes the head's CB tiles).
template <class K, class Args>
hipError_t launch_split(Args fa, hipStream_t st) {
  const SplitPlan p = split_plan(fa.d);
  return K::launch(fa, p.nfull, p.nhalf, p.unit_map, p.half_il, st);
}

// both parts in one launch
template <int DT, int LC, int NS>
struct FloatLaunch {
  static hipError_t launch(FusedFArgs fa, int64_t nfull, int64_t nhalf, bool unit_map, bool half_il,
                           hipStream_t st) {
    fa.nfull = nfull;
    fa.unit_map = unit_map;
    fa.half_il = half_il;
    const int64_t blocks = nfull + 2 * nhalf;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_fused_f16<DT, LC, NS>), dim3((unsigned)blocks), dim3(kThreads), 0, st, fa);
    return hipGetLastError();
  }
};

}  // namespace

// Compute units of the current device (0 when the runtime cannot say). Asked
// of the runtime on every call, so the library keeps no mutable state.
int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

bool fused_supported(const Dims& d, int dtype, bool int8) {
  // row strides (bytes) and the position index enter 24-bit multiplies
  if ((int64_t)d.H * d.P * 4 >= (1 << 24) || (int64_t)d.G * d.N * 4 >= (1 << 24)) return false;
  if (d.L >= (1 << 24)) return false;
  if (!int8) {
    if ((dtype != DT_F16 && dtype != DT_BF16) || d.P != kP) return false;
    if (d.N != 64 && d.N != 128) return false;
    if (d.l != 128 && d.l != 256) return false;
    if (d.B * d.H > (int64_t)1 << 30) return false;
    if (d.L * d.H * (int64_t)d.P * 2 >= ((int64_t)1 << 31)) return false;
    return d.L * d.G * (int64_t)d.N * 2 < ((int64_t)1 << 31);
  }
  // per-sequence offsets are formed in 32 bits
  if (d.L * d.H * (int64_t)d.P * 2 >= ((int64_t)1 << 31)) return false;
  if (d.B * d.G > 65535 || d.B * d.H > (int64_t)1 << 30) return false;
  if (dtype != DT_F16 && dtype != DT_BF16) return false;
  if (d.P != kP) return false;
  if (d.N != 64 && d.N != 128) return false;
  if (d.l != 128 && d.l != 256) return false;
  return true;
}

size_t fused_workspace_bytes(const Dims& d, bool int8) {
  if (int8) return fused_i8_workspace_bytes(d);
  return 2 * al((size_t)d.B * d.H * d.c * d.l * sizeof(float));
}

hipError_t launch_forward_fused(const Dims& d, int dtype, bool int8, const void* X,
                                const void* dt, const float* A, const void* B, const void* C,
                                const float* D, const ScalePtrs& sc, void* Y,
                                const void* initial_state, void* final_state, void* ws,
                                int8_t* tap_qxs, int32_t* tap_s32, int8_t* tap_s8,
                                int8_t* tap_passed, hipStream_t st) {
  if (!fused_supported(d, dtype, int8)) return hipErrorNotSupported;
  if (!int8) {
    const size_t cs = (size_t)d.B * d.H * d.c * d.l * sizeof(float);
    float* dAcs = (float*)ws;
    float* lut = (float*)((char*)ws + al(cs));
    hipError_t e = launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, nullptr, st);
    if (e != hipSuccess) return e;
    const FusedFArgs fa{d, X, dt, B, C, dAcs, lut, D, Y, (const float*)initial_state,
                        (float*)final_state, 0, 0, 0};
    if (dtype == DT_F16) {
      if (d.l == 256 && d.N == 128) return launch_split<FloatLaunch<DT_F16, 256, 128>>(fa, st);
      if (d.l == 256) return launch_split<FloatLaunch<DT_F16, 256, 64>>(fa, st);
      if (d.N == 128) return launch_split<FloatLaunch<DT_F16, 128, 128>>(fa, st);
      return launch_split<FloatLaunch<DT_F16, 128, 64>>(fa, st);
    }
    if (d.l == 256 && d.N == 128) return launch_split<FloatLaunch<DT_BF16, 256, 128>>(fa, st);
    if (d.l == 256) return launch_split<FloatLaunch<DT_BF16, 256, 64>>(fa, st);
    if (d.N == 128) return launch_split<FloatLaunch<DT_BF16, 128, 128>>(fa, st);
    return launch_split<FloatLaunch<DT_BF16, 128, 64>>(fa, st);
  }
  return launch_forward_i8(d, dtype, X, dt, A, B, C, D, sc, Y, initial_state, final_state, ws, tap_qxs, tap_s32,
                           tap_s8, tap_passed, st);
}

}  // namespace ssd
