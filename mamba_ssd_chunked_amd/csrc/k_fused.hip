// Fused SSD forward on the persistent-INT8 path ("SSDi8" notes page, "Overall
// framework" and "Key designs 1-3").
//
// A preparation launch quantises B and C once per group and forms the float64
// in-chunk cumulative sums (two launches when the combined grid would be too
// large). The main kernel runs one workgroup of eight waves per (batch, head). It walks that head's chunks in order and keeps the
// INT8 state in registers, so the state never travels through HBM. Per chunk:
//
//   Q(Xs)        X_scaled = LUT_state * x quantised once per (s, p) into LDS;
//   ChunkState   S32^T[n,p] = sum_s Q(B)^T[n,s] Q(Xs)[s,p]   (int8 MFMA; wave w
//                owns one n tile and its p tiles; Q(B)^T comes from the Q(B)
//                rows in LDS through transposing reads), requantised in
//                registers to S8;
//   ChunkScan1   Y_off[s,p] = sum_n Q(C)[s,n] H8_{k-1}[p,n]  (int8 MFMA, H8 in LDS);
//   ChunkBMM     CB^T tiles = Q(B) rows x Q(C) rows          (int8 MFMA; the output
//                lane layout is ChunkScan2's A-operand layout);
//   ChunkScan2   Y_diag = W x, W = CB s_C s_B exp(a_s - a_s') dt_s'  (fp16/bf16 MFMA);
//   StatePassing H8_k = sat(S8_k + RSH7(Q(Decay_k) H8_{k-1}))  (Eq. 6, in registers).
//
// Chunk k+1's x tile and per-position vectors are loaded into registers before
// chunk k's ChunkState and written to LDS after its scan; its Q(B) rows are
// then copied from memory straight into the freed LDS buffer and its Q(C) rows
// into registers, landing during the staging and StatePassing. HBM latency
// thus overlaps the MFMA/VALU work.
//
// ChunkScan2 factorisation (exact algebra): for a column tile j strictly below
// row tile i, exp(a_s - a_s') = u_s * V_i[s'] with u_s = exp(a_s - a_{16i}) <= 1
// and V_i[s'] = exp(a_{16i} - a_s') <= 1, so each row tile needs one table V_i
// and one factor per output row instead of an exponential per element.
// Off-diagonal tiles accumulate unscaled and are multiplied by u_s once; the
// diagonal tile uses exp(a_s - a_s') directly.
#include "ssd_cumsum.hpp"
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {
namespace {

constexpr int kP = 64;        // head dim of the fused kernel
constexpr int kThreads = 512;  // eight waves
constexpr int kWaves = kThreads / kWave;
// The INT8 kernel adds kProdWaves producer waves to the kWaves compute waves.
constexpr int kProdWaves = 4;
constexpr int kThreadsI8 = kThreads + kProdWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;

// 2^x with the hardware transcendental (arguments here are <= 0; results that
// would be denormal flush to 0, far below anything that reaches the output).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// LDS layouts. Rows are split into 16-byte chunks whose index is XOR-swizzled
// with low row bits, so the 8 or 16 lanes served together hit distinct banks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xsw(int p) { return (p ^ (p >> 3)) & 7; }
// x transposed, [p][s'] in 2-byte elements, with s reordered inside each block
// of 32 positions (two 16-position column tiles 2m and 2m + 1): the 4-position
// runs s = 32m + 16h + 4g + (0..3) sit at 32m + 8g + 4h + (0..3). A lane's
// ChunkScan2 operand (group g of tiles 2m and 2m + 1) is then one 16-byte
// chunk, index 4m + g. Rows are padded by 16 bytes (kXTPad elements), so 16
// consecutive rows start in 16 different bank groups, and the two low bits of
// the chunk index are XORed with bits 4-5 of the row, which spreads the
// staging's writes to rows 8 apart. For the operand reads, whose 16 rows
// share bits 4-5, the offset is then linear in m (no per-step swizzle).
constexpr int kXTPad = 8;
template <int LC>
__device__ __forceinline__ int xT_pair(int p, int m, int g) {  // 16-byte chunk start
  return p * (LC + kXTPad) + 32 * m + 8 * (g ^ ((p >> 4) & 3));  // = chunk (4m + g) ^ ((p >> 4) & 3)
}
template <int LC>
__device__ __forceinline__ int xT_off(int p, int s) {  // s aligned to 4
  return xT_pair<LC>(p, s >> 5, (s >> 2) & 3) + 4 * ((s >> 4) & 1);
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

// ---------------------------------------------------------------------------
// Prologue: Q(B), Q(C) with padded rows (t >= L -> 0), once per group. One
// block of NT threads quantises one 64-row x N tile: tile (bx, by) with bx over
// c * l / 64 row blocks and by over B * G.
// ---------------------------------------------------------------------------
template <int DT, int NT, int RB>  // RB rows of one chunk per block
__device__ __forceinline__ void prologue_bc_block(const Dims& d, const void* __restrict__ B,
                                                  const void* __restrict__ C,
                                                  const float* __restrict__ inv_B,
                                                  const float* __restrict__ inv_C,
                                                  int8_t* __restrict__ qB,
                                                  int8_t* __restrict__ qC, int bx, int64_t by) {
  const int nsb = d.l / RB;
  const int k = bx / nsb, sb = bx % nsb;
  const int64_t bg = by;
  const int64_t b = bg / d.G;
  const int g = (int)(bg % d.G);
  const int N = d.N, l = d.l;
  const int64_t Lp = (int64_t)d.c * l;
  const float ib = inv_B[g], ic = inv_C[g];
  // N <= 128, so a thread has at most RB * 16 / NT items; all their loads are
  // issued before any is used (rows past L read row L - 1 and are written as zeros)
  constexpr int kIt = RB * (128 / 8) / NT;
  float xb[kIt][8], xc[kIt][8];
#pragma unroll
  for (int u = 0; u < kIt; ++u) {
    const int item = (int)threadIdx.x + NT * u;
    if (item < RB * (N / 8)) {
      const int sl = item / (N / 8), n0 = (item % (N / 8)) * 8;
      const int64_t t = min((int64_t)k * l + RB * sb + sl, d.L - 1);
      const int64_t src = ((b * d.L + t) * d.G + g) * (int64_t)N + n0;
      ld8_f<DT>(B, src, xb[u]);
      ld8_f<DT>(C, src, xc[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kIt; ++u) {
    const int item = (int)threadIdx.x + NT * u;
    if (item >= RB * (N / 8)) break;
    const int sl = item / (N / 8), n0 = (item % (N / 8)) * 8;
    const int64_t t = (int64_t)k * l + RB * sb + sl;
    int qb[8], qc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qb[j] = t < d.L ? q_sat(xb[u][j] * ib, 127.f) : 0;
      qc[j] = t < d.L ? q_sat(xc[u][j] * ic, 127.f) : 0;
    }
    const int64_t dst = ((b * Lp + t) * d.G + g) * (int64_t)N + n0;
    *(uint2*)(qB + dst) = make_uint2(pack4(qb[0], qb[1], qb[2], qb[3]), pack4(qb[4], qb[5], qb[6], qb[7]));
    *(uint2*)(qC + dst) = make_uint2(pack4(qc[0], qc[1], qc[2], qc[3]), pack4(qc[4], qc[5], qc[6], qc[7]));
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_prologue_bc(Dims d, const void* __restrict__ B,
                                                     const void* __restrict__ C,
                                                     const float* __restrict__ inv_B,
                                                     const float* __restrict__ inv_C,
                                                     int8_t* __restrict__ qB,
                                                     int8_t* __restrict__ qC) {
  prologue_bc_block<DT, 256, 64>(d, B, C, inv_B, inv_C, qB, qC, blockIdx.x, blockIdx.y);
}

// The INT8 path's preparation in one launch: blocks [0, ncs) run ChunkCumsum
// (dAcs, LUT_state, Q(Decay)), the rest the B/C prologue, kPrepRows rows of a
// chunk each (chunks of 128 or 256). Both parts are short and latency-bound, so
// running them side by side hides one behind the other. Registers are capped so
// that two blocks share a CU: for the 2.7B layer (b 8, L 2048, 80 heads) the
// whole grid of 448 blocks is then resident at once.
constexpr int kPrepRows = 128;
template <int DT>
__global__ __launch_bounds__(kCsThreads) __attribute__((amdgpu_waves_per_eu(8))) void k_prep_i8(Dims d, const void* __restrict__ dt,
                                                 const float* __restrict__ A,
                                                 float* __restrict__ dAcs, float* __restrict__ lut,
                                                 uint8_t* __restrict__ qdecay,
                                                 const void* __restrict__ B,
                                                 const void* __restrict__ C,
                                                 const float* __restrict__ inv_B,
                                                 const float* __restrict__ inv_C,
                                                 int8_t* __restrict__ qB, int8_t* __restrict__ qC,
                                                 int ncs) {
  const int bi = blockIdx.x;
  if (bi < ncs) {
    // ChunkCumsum block (k, b, head block) from the linear index
    const int k = bi % d.c;
    const int rest = bi / d.c;
    const int64_t b = rest % d.B;
    chunk_cumsum_block<DT>(dt, A, dAcs, lut, qdecay, d, k, b, (int)(rest / d.B));
  } else {
    const int pi = bi - ncs;
    const int nbx = d.c * (d.l / kPrepRows);
    prologue_bc_block<DT, kCsThreads, kPrepRows>(d, B, C, inv_B, inv_C, qB, qC, pi % nbx, pi / nbx);
  }
}

// ---------------------------------------------------------------------------
// Block -> head. Slots 0 .. B*H - 1 list every head once. With unit_map
// ((B*G) % 8 == 0) slot s serves unit (s % 8) + 8 ((s / 8) / hpg), head
// (s / 8) % hpg of that unit (unit = batch * G + group), so slots on one XCD
// (block i runs on XCD i % 8) cover whole units and the int8 B/C rows of a
// unit stay in one XCD's L2; otherwise slot s is unit s / hpg. Whole-head
// blocks [0, nfull) take slot = block. The p-half blocks after them take slots
// nfull .. B*H - 1, two blocks per slot: with half_il (nfull and the half count
// both multiples of 8) block nfull + bx takes slot nfull + bx % 8 + 8 (j / 2)
// and half j % 2 (j = bx / 8), so it runs on its slot's XCD; otherwise slot
// nfull + bx / 2 and half bx % 2. One slot map serves both parts, so every
// head is computed exactly once.
// ---------------------------------------------------------------------------
struct BlockHead {
  int64_t unit, hl;
  int ph;
};
template <int PW>
__device__ __forceinline__ BlockHead block_head(const Dims& d, int64_t bx, int64_t nfull, int unit_map,
                                                int half_il) {
  BlockHead r;
  int64_t slot;
  r.ph = 0;
  if (PW == 4) {
    slot = bx;
  } else if (half_il) {
    const int64_t j = bx / 8;
    slot = nfull + (bx % 8) + 8 * (j >> 1);
    r.ph = (int)(j & 1);
  } else {
    slot = nfull + bx / 2;
    r.ph = (int)(bx & 1);
  }
  if (unit_map) {
    const int64_t j = slot / 8;
    r.unit = (slot % 8) + 8 * (j / d.hpg);
    r.hl = j % d.hpg;
  } else {
    r.unit = slot / d.hpg;
    r.hl = slot % d.hpg;
  }
  return r;
}

// ---------------------------------------------------------------------------
// main fused kernel
// ---------------------------------------------------------------------------
struct FusedArgs {
  Dims d;
  const void* X;
  const void* dt;
  const int8_t* qB;
  const int8_t* qC;
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
  // launch layout: blocks [0, nfull) run whole heads (slots 0 .. nfull - 1), the
  // rest run p halves of heads nfull .. (two blocks per head)
  int64_t nfull;
  int unit_map;  // slot -> head map that keeps whole (batch, group) units on one XCD
  int half_il;   // the p-half blocks are interleaved by 8 (see block_head)
};

// The LDS arrays of one chunk buffer of the INT8 kernel.
template <int LC, int NS>
struct Smem {
  u16* xT;      // x^T [p][s], 2-byte elements (swizzled, see xT_pair)
  int8_t* qB;   // Q(B) rows [s][n] (swizzled, see b_off)
  int8_t* qx;   // Q(X_scaled)^T [p][s] (swizzled, see qx_off)
  int8_t* h8;   // passed state [p][n]
  float* vec;   // a * log2(e) [l], dt [l]
  float* vw;    // one ChunkScan2 table per wave [l]
  float* ss;    // s_S[h, p], inv_X[h, p], M_req[h, p]
};

// Q(X_scaled)^T tile [p][s] (bytes); s aligned to 4
template <int LC>
__device__ __forceinline__ int qx_off(int p, int s) {
  return p * LC + 16 * ((s >> 4) ^ xsw(p)) + (s & 15);
}

// Registers holding one staging item of a chunk: item it = (q = it / C8N, c8 =
// it % C8N) owns x rows 4q .. 4q+3 at p = 8 c8 .. 8 c8 + 7, plus the
// per-position vectors of position it % l. Every load is unconditional
// (addresses are clamped into the tensor and out-of-range rows are zeroed when
// stored to LDS).
template <int LC, int NS, int PW>
struct Prefetch {
  static constexpr int C8N = 2 * PW;          // 8-column groups of p per workgroup
  static constexpr int XI = (LC / 4) * C8N;
  static_assert(XI <= kThreads, "tile split");
  uint4 x[4];
  float4 lut;
  float va;     // dAcs (scaled by log2(e) when stored)
  uint32_t vd;  // dt bits in the input type (converted when stored)
};

// Per-item byte offsets of the staging loads (the per-chunk parts are
// wave-uniform and live in scalar registers).
template <int LC, int NS, int PW>
struct LaneOff {
  uint32_t q4;   // first x row of this item (4q)
  uint32_t xc;   // byte offset of columns 8 c8 .. 8 c8 + 7 within a row
  uint32_t lut;  // lut / dAcs entries 4q .. 4q + 3
  uint32_t sv;   // position of the per-position vectors (dAcs, dt)
};

template <int DT, int LC, int NS, int PW>
__device__ __forceinline__ LaneOff<LC, NS, PW> lane_offsets(const Dims& d, int tid, int c8base) {
  typedef typename Store<DT>::T T;
  typedef Prefetch<LC, NS, PW> PF;
  typedef LaneOff<LC, NS, PW> LO;
  LO o;
  const int it = tid % PF::XI;
  const int q = it / PF::C8N, c8 = c8base + it % PF::C8N;
  o.q4 = (uint32_t)(4 * q);
  o.xc = (uint32_t)(8 * c8 * (int)sizeof(T));
  o.lut = (uint32_t)(16 * q);
  o.sv = (uint32_t)(tid % LC);
  return o;
}

template <int DT, int LC, int NS, int PW>
__device__ __forceinline__ void prefetch_load(const FusedArgs& a, int64_t b, int h, int k, int tid,
                                              int c8base, const LaneOff<LC, NS, PW>& lo,
                                              Prefetch<LC, NS, PW>& pf) {
  typedef typename Store<DT>::T T;
  typedef Prefetch<LC, NS, PW> PF;
  const Dims& d = a.d;
  // wave-uniform 64-bit bases plus per-lane 32-bit offsets (one sequence of x is
  // below 2 GB, checked by fused_supported)
  const int t0 = k * LC;
  const int64_t cs0 = ((b * d.H + h) * d.c + k) * (int64_t)LC;
  const int64_t rowB = (int64_t)d.H * kP * sizeof(T);  // bytes per position of x
  const char* xk = (const char*)a.X + (b * d.L * d.H + h) * (int64_t)kP * sizeof(T) + t0 * rowB;
  const char* dtk = (const char*)a.dt + ((b * d.L + t0) * d.H + h) * (int64_t)sizeof(T);
  // positions past L (ragged last chunk) read row L - 1; the clamp is a min,
  // not a branch, so no load has to complete before the chunk's compute
  const uint32_t lim = (uint32_t)min((int64_t)LC - 1, d.L - 1 - t0);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    pf.x[r] = *(const uint4*)(xk + (__umul24(min(lo.q4 + r, lim), rowB) + lo.xc));
  if constexpr (sizeof(T) == 4)
    pf.vd = *(const uint32_t*)(dtk + min(lo.sv, lim) * (uint32_t)(d.H * sizeof(T)));
  else
    pf.vd = *(const u16*)(dtk + __umul24(min(lo.sv, lim), (uint32_t)(d.H * sizeof(T))));
  pf.lut = *(const float4*)((const char*)(a.lut + cs0) + lo.lut);
  pf.va = *(const float*)((const char*)(a.dAcs + cs0) + 4 * lo.sv);
}

typedef int v2i __attribute__((ext_vector_type(2)));
// Transposing LDS read (8-bit elements): the 16 lanes of a group each point at
// 8 bytes; lanes 2r and 2r + 1 form row r (16 bytes) of an 8 x 16 byte matrix,
// and lane i receives column i, i.e. byte i of every row.
__device__ __forceinline__ v2i lds_tr8(const int8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(int8_t*)p);
}

// Writes the prefetched chunk into LDS: x transposed, Q(X_scaled) =
// sat(RHAZ(fl32(fl32(lut * x) * inv_X))) transposed (the quantiser of "Key
// design 1") and the per-position vectors.
template <int DT, int LC, int NS, int PW, bool TAPS>
__device__ __forceinline__ void prefetch_store(const FusedArgs& a, const Smem<LC, NS>& sm, int64_t b, int h, int k,
                                               int tid, int c8base, const Prefetch<LC, NS, PW>& pf) {
  typedef typename Store<DT>::T T;
  typedef Prefetch<LC, NS, PW> PF;
  const int t0 = k * LC;
  // Every prefetched register passes through an empty asm here, in all lanes:
  // nothing that uses the values (unpacking, conversion) can then be scheduled
  // right after the loads, which would make the prefetch wait for memory; and
  // no lane leaves the staging below with a load still outstanding (a lane that
  // skipped a branch would carry one, and where the paths merge the compiler
  // would then wait for every outstanding load, the next chunk's Q(B) copies
  // and Q(C) rows included).
  uint4 xr[4] = {pf.x[0], pf.x[1], pf.x[2], pf.x[3]};
#pragma unroll
  for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(xr[r].x), "+v"(xr[r].y), "+v"(xr[r].z), "+v"(xr[r].w));
  float4 lutp = pf.lut;
  float vap = pf.va;
  uint32_t vdp = pf.vd;
  asm volatile("" : "+v"(lutp.x), "+v"(lutp.y), "+v"(lutp.z), "+v"(lutp.w), "+v"(vap), "+v"(vdp));
  if (tid < PF::XI) {
    const int q = tid / PF::C8N, c8 = c8base + tid % PF::C8N;
    // Rows past L (ragged last chunk) hold copies of row L-1 (finite values):
    // their LUT_state is 0, so their Q(X_scaled) is 0, and ChunkScan2 never
    // pairs them with a valid output row (causal mask) and gives them weight 0.
    const uint32_t* w0 = (const uint32_t*)&xr[0];
    const uint32_t* w1 = (const uint32_t*)&xr[1];
    const uint32_t* w2 = (const uint32_t*)&xr[2];
    const uint32_t* w3 = (const uint32_t*)&xr[3];
    // x^T: s = 4q sits in 16-byte chunk 4 (q >> 3) + (q & 3), half (q >> 2) & 1;
    // the rows p = 8 c8 + e' share bits 4-5 (c8 >> 1), so one base serves all 8
    u16* const xTb = sm.xT + xT_pair<LC>(8 * c8, q >> 3, q & 3) + 4 * ((q >> 2) & 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // dword e of each row holds p = 8 c8 + 2e (low half) and 2e + 1 (high half)
      const uint32_t lo01 = __builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(w1[e], w0[e], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(w3[e], w2[e], 0x07060302u);
      *(uint2*)(xTb + (2 * e) * (LC + kXTPad)) = make_uint2(lo01, lo23);
      *(uint2*)(xTb + (2 * e + 1) * (LC + kXTPad)) = make_uint2(hi01, hi23);
    }
    const float lutv[4] = {lutp.x, lutp.y, lutp.z, lutp.w};
    const float* ixl = sm.ss + kP + 8 * c8;
    const float4 i0 = *(const float4*)ixl, i1 = *(const float4*)(ixl + 4);
    const float invx8[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
    // Q(X_scaled)^T: for p = 8 c8 + e the swizzle is e ^ c8; s = 4q is byte
    // 4 (q & 3) of 16-byte chunk (q >> 2) ^ xsw(p)
    char* qxb = (char*)sm.qx + 8 * LC * c8 + 4 * (q & 3);
    const int qc = (q >> 2) ^ c8;
    uint32_t qd4[8];  // byte r: row 4q + r
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // fl32(lut * x) (one rounding; with fp16 x a single mixed-precision fma
        // with a zero addend), then fl32(. * inv_X)
        const uint32_t dw = (e >> 1) == 0 ? xr[r].x : (e >> 1) == 1 ? xr[r].y : (e >> 1) == 2 ? xr[r].z : xr[r].w;
        const uint32_t hv = (e & 1) ? (dw >> 16) : (dw & 0xffffu);
        const float xs = __builtin_fmaf(lutv[r], Store<DT>::to_f(__builtin_bit_cast(T, (u16)hv)), 0.0f);
        v[r] = xs * invx8[e];
      }
      qd4[e] = q8x4(v[0], v[1], v[2], v[3]);
      *(uint32_t*)(qxb + e * LC + 16 * (qc ^ e)) = qd4[e];
    }
    if (TAPS && a.tap_qxs) {
      const Dims& d = a.d;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = (int64_t)t0 + 4 * q + r;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo |= ((qd4[e] >> (8 * r)) & 0xffu) << (8 * e);
          hi |= ((qd4[e + 4] >> (8 * r)) & 0xffu) << (8 * e);
        }
        if (t < d.L) *(uint2*)(a.tap_qxs + ((b * d.L + t) * d.H + h) * (int64_t)kP + 8 * c8) = make_uint2(lo, hi);
      }
    }
  }
  if (tid < LC) {
    float* vec = sm.vec;
    vec[tid] = vap * kLog2e;
    float dtv;
    if constexpr (sizeof(T) == 4)
      dtv = __uint_as_float(vdp);
    else
      dtv = Store<DT>::to_f(__builtin_bit_cast(T, (u16)vdp));
    vec[LC + tid] = (t0 + tid < (int)a.d.L) ? dtv : 0.f;
  }
}

// PW = 4: the workgroup owns a whole head (all four 16-wide p tiles).
// PW = 2: it owns p tiles 2 ph, 2 ph + 1 of a head; two such workgroups cover
// the head, each recomputing the head's CB tiles. Used for the last, partial
// round of heads so that it spreads over every CU.
// TAPS: the instantiation that can write the debug taps (the others carry no
// tap code, which keeps their scalar registers free).
template <int DT, int LC, int NS, int PW, bool TAPS>
__device__ __forceinline__ void fused_i8_body(const FusedArgs& a, const int64_t bx, u16* s_xT, int8_t* s_qB,
                                              int8_t* s_qx, int8_t* s_h8, float* s_vec, float* s_vw,
                                              float* s_ss) {
  typedef typename Store<DT>::T T;
  typedef Prefetch<LC, NS, PW> PF;
  constexpr int RT = LC / 16;      // row tiles of the chunk
  constexpr int NT = NS / 16;      // n tiles of the state
  constexpr int PTW = PW * NT / kWaves;  // p tiles per wave in ChunkState / StatePassing
  constexpr int KS = LC / 64;      // ChunkState K steps
  constexpr int KN = NS / 64;      // K steps over N

  // x^T, Q(Xs)^T and the per-position vectors are double buffered: chunk k
  // computes from buffer k & 1 while the producer waves stage chunk k + 1 into
  // the other; the Q(B) rows (single buffer) are written between the two
  // barriers of a chunk
  constexpr int XTN = kP * (LC + kXTPad), QXN = kP * LC, VN = 2 * LC;
  const auto smem = [&](int kc) {
    const int o = kc & 1;
    return Smem<LC, NS>{s_xT + o * XTN, s_qB, s_qx + o * QXN, s_h8, s_vec + o * VN, s_vw, s_ss};
  };
  int8_t* H8l = s_h8;
  const int8_t* qBl = s_qB;
  float* SSl = s_ss;

  const Dims& d = a.d;
  // bx: the block's index within its part of the launch
  const BlockHead bh = block_head<PW>(d, bx, a.nfull, a.unit_map, a.half_il);
  const int64_t unit = bh.unit, hl = bh.hl;
  const int ph = bh.ph;
  const int pt_base = (PW == 4) ? 0 : 2 * ph;  // first p tile of this workgroup
  const int64_t b = unit / d.G;
  const int g_h = (int)(unit % d.G);
  const int h = g_h * d.hpg + (int)hl;
  const int w = wave_id();  // compute waves 0 .. kWaves - 1, then the producers
  const bool producer = w >= kWaves;
  const int ptid = (int)threadIdx.x - kThreads;  // producer thread index
  const int64_t Lp = (int64_t)d.c * LC;
  const int H = d.H;
  T* const ybase = (T*)a.Y + (b * d.L * H + h) * (int64_t)kP;  // uniform

  // ChunkState / StatePassing role: n tile nt_own, p tiles pt0 .. pt0 + PTW - 1
  // (each Q(B)^T row is read by exactly one wave)
  const int nt_own = w % NT;
  const int pt0 = pt_base + (w / NT) * PTW;
  const float scBC = a.sc.s_C[g_h] * a.sc.s_B[g_h];
  const float sC = a.sc.s_C[g_h];
  const float Dh = a.D[h];
  const int tid0 = threadIdx.x;
  if (tid0 < kP) {
    SSl[tid0] = a.sc.s_S[h * kP + tid0];
    SSl[kP + tid0] = a.sc.inv_X[h * kP + tid0];
    SSl[2 * kP + tid0] = a.sc.M_req[h * kP + tid0];
  }
  __syncthreads();
  float* Vw = s_vw + w * LC;

  uint32_t H8[PTW];  // passed state: lane (p = 16 (pt0 + j) + lane % 16, n = 16 nt_own + 4 (lane / 16) + r)
  const bool has_init = a.init != nullptr;
  if (!producer) {
    const int l16 = tid0 & 15, lg = (tid0 & (kWave - 1)) >> 4;
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int p = 16 * (pt0 + j) + l16;
      H8[j] = has_init ? *(const uint32_t*)(a.init + ((b * H + h) * (int64_t)kP + p) * NS + 16 * nt_own + 4 * lg)
                       : 0u;
      // the initial state feeds chunk 0's ChunkScan1
      if (has_init) *(uint32_t*)&H8l[b_off<NS>(p, 16 * nt_own + 4 * lg)] = H8[j];
    }
  }

  // Q(C) rows (B operand over N) of row tile {w, 15 - w}[rr] of chunk k (compute waves)
  const auto load_qc = [&](int k, int lane, int rr, v4i (&qc)[KN]) {
    const int8_t* qcb = a.qC + ((b * Lp + (int64_t)k * LC) * d.G + g_h) * (int64_t)NS;  // uniform
    const int l16 = lane & 15, lg = lane >> 4;
    const int i = min((rr == 0) ? w : 2 * kWaves - 1 - w, RT - 1);
    const int8_t* src = qcb + (__umul24(16 * i + l16, d.G * NS) + 16 * lg);
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) qc[kn] = *(const v4i*)(src + 64 * kn);
  };
  // the dword holding Q(Decay) of chunk k
  const auto load_qd = [&](int k) {
    const int64_t qi = (b * H + h) * d.c + k;
    return *(const uint32_t*)(a.qdecay + (qi & ~(int64_t)3));
  };

  // Producer side: thread ptid stages x items ptid + 256 u (u < NIT, items
  // below XI) and copies the Q(B) rows through registers, 16 bytes x QBN per
  // thread. (XI >= l, so the threads that store the per-position vectors,
  // ptid < l, all have an item.)
  constexpr int NPT = kProdWaves * kWave;
  constexpr int NIT = (PF::XI + NPT - 1) / NPT;
  static_assert(PF::XI >= LC && (PF::XI % NPT == 0 || PF::XI < NPT), "producer split");
  constexpr int QBN = LC * NS / 16 / NPT;
  static_assert(QBN >= 1, "Q(B) split");
  const auto qb_src = [&](int kc, int v) {  // Q(B) row chunk ptid + 256 v of chunk kc
    const int ci = ptid + NPT * v;
    const int r = ci / (NS / 16), c16 = ci % (NS / 16);
    return a.qB + ((b * Lp + (int64_t)kc * LC + r) * d.G + g_h) * (int64_t)NS + 16 * c16;
  };
  // (the register arrays are passed as arguments, not captured, so they stay in
  // registers)
  const auto produce_load = [&](int kc, PF (&pfs)[NIT], v4i (&qbr)[QBN]) {  // issue every load of chunk kc
#pragma unroll
    for (int v = 0; v < QBN; ++v) qbr[v] = *(const v4i*)qb_src(kc, v);
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
      const int it = ptid + NPT * u;
      if (it < PF::XI) {
        const LaneOff<LC, NS, PW> lo = lane_offsets<DT, LC, NS, PW>(d, it, 2 * pt_base);
        prefetch_load<DT, LC, NS, PW>(a, b, h, kc, it, 2 * pt_base, lo, pfs[u]);
      }
    }
  };
  const auto produce_stage = [&](int kc, const PF (&pfs)[NIT]) {  // x^T, Q(Xs)^T, vectors of chunk kc into buffer kc & 1
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int u = 0; u < NIT; ++u)
      if (ptid + NPT * u < PF::XI)
        prefetch_store<DT, LC, NS, PW, TAPS>(a, smem(kc), b, h, kc, ptid + NPT * u, 2 * pt_base, pfs[u]);
  };
  const auto produce_qb = [&](const v4i (&qbr)[QBN]) {  // the Q(B) rows into LDS (b_off layout)
#pragma unroll
    for (int v = 0; v < QBN; ++v) {
      const int ci = ptid + NPT * v;
      const int r = ci / (NS / 16), c16 = ci % (NS / 16);
      *(v4i*)(s_qB + b_off<NS>(r, 16 * c16)) = qbr[v];
    }
  };

  if (producer) {
    // The producer waves run their own loop, with the same two barriers per
    // chunk as the compute waves' loop below (so no value of one role is live
    // in the other's loop).
    PF pfs[NIT];
    v4i qbr[QBN];  // (a vector type: struct copies would keep the array in scratch)
    produce_load(0, pfs, qbr);
    produce_stage(0, pfs);
    produce_qb(qbr);
    for (int k = 0; k < d.c; ++k) {
      __syncthreads();  // chunk k staged (B1)
      if (k + 1 < d.c) {
        produce_load(k + 1, pfs, qbr);
        produce_stage(k + 1, pfs);
      }
      __syncthreads();  // chunk k's Q(B) rows no longer read (B2)
      if (k + 1 < d.c) produce_qb(qbr);
    }
    return;
  }

  v4i qc2[2][KN];
  load_qc(0, tid0 & (kWave - 1), 0, qc2[0]);
  load_qc(0, tid0 & (kWave - 1), 1, qc2[1]);
  uint32_t qd_cur = load_qd(0);  // dword holding Q(Decay) of the current chunk

  for (int k = 0; k < d.c; ++k) {
    // Lane indices re-derived from an opaque copy every chunk: the swizzled LDS
    // offsets built from them are then recomputed (a few VALU operations)
    // instead of being hoisted out of the loop and spilled.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int l16 = lane & 15, lg = lane >> 4;
    const int64_t t0 = (int64_t)k * LC;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's Q(C) rows and Q(Decay) have landed
    __syncthreads();  // chunk k staged (x^T, Q(Xs), vectors, Q(B)); H8l holds H_{k-1}
    // The next chunk's loads are issued unconditionally (the last chunk reloads
    // itself): with no branch around them the compiler counts outstanding loads
    // exactly instead of waiting for all of them where the paths merge.
    const int kn = min(k + 1, d.c - 1);
    const Smem<LC, NS> sm = smem(k);
    const u16* xT = sm.xT;
    const int8_t* qxl = sm.qx;
    const float* vA2 = sm.vec;
    const float* vDt = vA2 + LC;
    v2s S8a[PTW], S8b[PTW];  // local state codes n = 4 lg + {0, 1} and {2, 3} of each dword
    v4i qcn1[KN];            // Q(C) rows of row tile 15 - w of the next chunk
    // The Q(C) rows are complete (they were loaded during the previous chunk);
    // passing them through an empty asm here keeps the compiler from placing its
    // own wait for them inside the scan loops.
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int q = 0; q < KN; ++q) asm volatile("" : "+v"(qc2[rr][q]));
    load_qc(kn, lane, 1, qcn1);
    const uint32_t qd_next = load_qd(kn);

    // ---- ChunkState^T for (n tile nt_own, p tiles pt0 ..) ----
    {
      v4i acc[PTW];
      // A operand Q(B)^T[n, s] straight from the Q(B) rows with two transposing
      // reads: lane (lg, l16) gets n = 16 nt_own + l16 and s = s0 .. s0 + 15.
      // The operands of step ks + 1 are read while step ks multiplies.
      const int cB = 16 * nt_own + 8 * (l16 & 1);
      v4i qa[2], bq[2][PTW];
      const auto load_ks = [&](int ks, v4i& a_, v4i (&b_)[PTW]) {
        const int s0 = 64 * ks + 16 * lg;
        const v2i lo = lds_tr8(qBl + b_off<NS>(s0 + (l16 >> 1), cB));
        const v2i hi = lds_tr8(qBl + b_off<NS>(s0 + 8 + (l16 >> 1), cB));
        a_ = v4i{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int j = 0; j < PTW; ++j) b_[j] = *(const v4i*)&qxl[qx_off<LC>(16 * (pt0 + j) + l16, s0)];
      };
      load_ks(0, qa[0], bq[0]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) load_ks(ks + 1, qa[(ks + 1) & 1], bq[(ks + 1) & 1]);
#pragma unroll
        for (int j = 0; j < PTW; ++j)
          acc[j] = mma_i8(qa[ks & 1], bq[ks & 1][j], ks == 0 ? v4i{0, 0, 0, 0} : acc[j]);
      }
#pragma unroll
      for (int j = 0; j < PTW; ++j) {
        const int p = 16 * (pt0 + j) + l16;
        if (TAPS && a.tap_s32) {
          const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kP + p) * NS + 16 * nt_own + 4 * lg;
          *(int4*)(a.tap_s32 + so) = make_int4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
        }
        // requantise in registers (Key design 2); the codes stay as int16 pairs
        // for the packed Eq. 6 update
        const float mreq = SSl[2 * kP + p];
        S8a[j] = cvt_pair(q8_pre((float)acc[j][0] * mreq), q8_pre((float)acc[j][1] * mreq));
        S8b[j] = cvt_pair(q8_pre((float)acc[j][2] * mreq), q8_pre((float)acc[j][3] * mreq));
      }
    }

    // ---- ChunkScan, transposed: Y^T[p, s] for row tiles {w, 15 - w} ----
    // (outputs land as 4 consecutive p per lane for one position s)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      // l = 256: tiles w and 15 - w (balanced under the causal mask); l = 128: tile w
      const int i = (rr == 0) ? w : 2 * kWaves - 1 - w;
      if (i >= RT) continue;
      const int s_row = 16 * i + l16;   // this lane's position s (B-operand column)
      v4i qcr[KN];  // (selected, not indexed, so qc2 stays in registers)
#pragma unroll
      for (int kn = 0; kn < KN; ++kn) qcr[kn] = rr ? qc2[1][kn] : qc2[0][kn];
      // V_i[s'] = s_C s_B exp(a_{16i} - a_s') dt_s' for s' < 16 i (this wave's table)
      const float a_ref = vA2[16 * i];
      for (int sp = lane; sp < 16 * i; sp += kWave) Vw[sp] = scBC * fast_exp2(a_ref - vA2[sp]) * vDt[sp];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // one accumulator per p tile: off-diagonal tiles are summed unscaled, then
      // multiplied by u_s; ChunkScan1 and the diagonal tile add on top
      v4f acc[PW];
      // off-diagonal column tiles j < i in full pairs (jA, jA + 1); the first
      // pair starts the accumulators (zero addend) instead of a separate clear
      const auto pair = [&](int jA, bool first) {
        const int jB = jA + 1;
        v4i ba[KN], bb[KN];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          ba[kn] = *(const v4i*)&qBl[b_off<NS>(16 * jA + l16, 64 * kn + 16 * lg)];
          bb[kn] = *(const v4i*)&qBl[b_off<NS>(16 * jB + l16, 64 * kn + 16 * lg)];
        }
        const float4 vA = *(const float4*)&Vw[16 * jA + 4 * lg];
        const float4 vB = *(const float4*)&Vw[16 * jB + 4 * lg];
        FragF<DT> xf[PW];
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) xf[jp] = frag16<DT>(&xT[xT_pair<LC>(16 * (pt_base + jp) + l16, jA >> 1, lg)]);
        v4i cbA = v4i{0, 0, 0, 0}, cbB = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          cbA = mma_i8(ba[kn], qcr[kn], cbA);
          cbB = mma_i8(bb[kn], qcr[kn], cbB);
        }
        FragF<DT> wf;
        wf.set(0, (float)cbA[0] * vA.x);
        wf.set(1, (float)cbA[1] * vA.y);
        wf.set(2, (float)cbA[2] * vA.z);
        wf.set(3, (float)cbA[3] * vA.w);
        wf.set(4, (float)cbB[0] * vB.x);
        wf.set(5, (float)cbB[1] * vB.y);
        wf.set(6, (float)cbB[2] * vB.z);
        wf.set(7, (float)cbB[3] * vB.w);
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) acc[jp] = FragF<DT>::mma(xf[jp], wf, first ? v4f{0, 0, 0, 0} : acc[jp]);
      };
      if (i >= 2) {
        pair(0, true);
        for (int jA = 2; jA + 1 < i; jA += 2) pair(jA, false);
      } else {
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) acc[jp] = v4f{0, 0, 0, 0};
      }
      // diagonal tile j = i (with D on its diagonal, so the skip term D x rides the
      // MFMA). It shares its MFMA with the other tile of its pair (2m, 2m + 1),
      // m = i / 2: for odd i that is the leftover off-diagonal tile i - 1, whose
      // weights carry u_s so it can join the unscaled diagonal accumulator; for
      // even i it is tile i + 1, above the diagonal, with zero weights.
      const float a_s = vA2[s_row];
      const float us = fast_exp2(a_s - a_ref);  // u at this lane's position
#pragma unroll
      for (int jp = 0; jp < PW; ++jp) acc[jp] *= us;
      // ChunkScan1 (inter-chunk), transposed: H8 rows x Q(C) rows, scaled by
      // exp(a_s) s_C s_S[p] and added to the output accumulator. All operands
      // are read first and the MFMAs of the p tiles interleave, so the tiles'
      // LDS and MFMA latencies overlap instead of adding up.
      if (k > 0 || has_init) {
        const float eo = fast_exp2(a_s) * sC;
        v4i hb[KN][PW];
        float4 ssv[PW];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn)
#pragma unroll
          for (int jp = 0; jp < PW; ++jp)
            hb[kn][jp] = *(const v4i*)&H8l[b_off<NS>(16 * (pt_base + jp) + l16, 64 * kn + 16 * lg)];
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) ssv[jp] = *(const float4*)&SSl[16 * (pt_base + jp) + 4 * lg];
        v4i acc1[PW];
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) acc1[jp] = mma_i8(hb[0][jp], qcr[0], v4i{0, 0, 0, 0});
#pragma unroll
        for (int kn = 1; kn < KN; ++kn)
#pragma unroll
          for (int jp = 0; jp < PW; ++jp) acc1[jp] = mma_i8(hb[kn][jp], qcr[kn], acc1[jp]);
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) {
          acc[jp][0] = fmaf((float)acc1[jp][0], eo * ssv[jp].x, acc[jp][0]);
          acc[jp][1] = fmaf((float)acc1[jp][1], eo * ssv[jp].y, acc[jp][1]);
          acc[jp][2] = fmaf((float)acc1[jp][2], eo * ssv[jp].z, acc[jp][2]);
          acc[jp][3] = fmaf((float)acc1[jp][3], eo * ssv[jp].w, acc[jp][3]);
        }
      }
      {
        const int hd = i & 1;            // half of the pair holding the diagonal tile
        const int jL = i - 1;            // leftover tile (odd i only)
        v4i bd[KN], bl[KN];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          bd[kn] = *(const v4i*)&qBl[b_off<NS>(16 * i + l16, 64 * kn + 16 * lg)];
          if (hd) bl[kn] = *(const v4i*)&qBl[b_off<NS>(16 * jL + l16, 64 * kn + 16 * lg)];
        }
        const float4 ad = *(const float4*)&vA2[16 * i + 4 * lg];
        const float4 dd = *(const float4*)&vDt[16 * i + 4 * lg];
        float4 vL = make_float4(0.f, 0.f, 0.f, 0.f);
        if (hd) vL = *(const float4*)&Vw[16 * jL + 4 * lg];
        FragF<DT> xf[PW];
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) xf[jp] = frag16<DT>(&xT[xT_pair<LC>(16 * (pt_base + jp) + l16, i >> 1, lg)]);
        v4i cbD = v4i{0, 0, 0, 0}, cbL = v4i{0, 0, 0, 0};
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
          cbD = mma_i8(bd[kn], qcr[kn], cbD);
          if (hd) cbL = mma_i8(bl[kn], qcr[kn], cbL);
        }
        const float adv[4] = {ad.x, ad.y, ad.z, ad.w};
        const float ddv[4] = {dd.x, dd.y, dd.z, dd.w};
        const float vLv[4] = {vL.x * us, vL.y * us, vL.z * us, vL.w * us};
        float wd[4], wl[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sp = 16 * i + 4 * lg + r;
          // evaluated in every lane and then selected (no branch); above the
          // diagonal the exponent is positive and the discarded value may be inf
          const float wv = (float)cbD[r] * scBC * fast_exp2(a_s - adv[r]) * ddv[r];
          wd[r] = (sp < s_row) ? wv : (sp == s_row) ? wv + Dh : 0.f;
          wl[r] = (float)cbL[r] * vLv[r];
        }
        FragF<DT> wf;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          wf.set(r, hd ? wl[r] : wd[r]);
          wf.set(r + 4, hd ? wd[r] : 0.f);
        }
#pragma unroll
        for (int jp = 0; jp < PW; ++jp) acc[jp] = FragF<DT>::mma(xf[jp], wf, acc[jp]);
      }
      // epilogue: lane holds s = s_row and p = 16 pt + 4 lg + r
      const int64_t t = t0 + s_row;
      char* yrow = (char*)ybase + (__umul24((uint32_t)t, H * kP * (int)sizeof(T)) + 4 * lg * (int)sizeof(T));
#pragma unroll
      for (int jp = 0; jp < PW; ++jp) {
        const int pt = pt_base + jp;
        const float y[4] = {acc[jp][0], acc[jp][1], acc[jp][2], acc[jp][3]};
        if (t < d.L) *(uint2*)(yrow + 16 * pt * (int)sizeof(T)) = make_uint2(pack2<DT>(y[0], y[1]), pack2<DT>(y[2], y[3]));
      }
      __builtin_amdgcn_wave_barrier();  // this wave's table is rewritten by its next row tile
      if (rr == 0) load_qc(kn, lane, 0, qc2[0]);  // row tile w of the next chunk
    }
    __syncthreads();  // chunk k's tiles, Q(B) rows and H8l are no longer read; chunk k + 1 staged (B2)

    // ---- StatePassing (Eq. 6) in registers; publish H8 for the next ChunkScan1 ----
    const int qd = (int)((qd_cur >> (8 * (((b * H + h) * d.c + k) & 3))) & 0xff);
    const v2s qd2 = {(short)qd, (short)qd};
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int p = 16 * (pt0 + j) + l16;
      if (k == 0 && !has_init) {
        H8[j] = pack_pairs(S8a[j], S8b[j]);
      } else {
        // two elements per lane op: RSH7 of the int16 products, add, saturate
        const v2s r01 = rsh7_pair(qd2, unpack_pair(H8[j], 0x010c000cu));
        const v2s r23 = rsh7_pair(qd2, unpack_pair(H8[j], 0x030c020cu));
        H8[j] = pack_pairs(sat127_pair(S8a[j] + r01), sat127_pair(S8b[j] + r23));
      }
      *(uint32_t*)&H8l[b_off<NS>(p, 16 * nt_own + 4 * lg)] = H8[j];
      const int64_t so = (((b * d.c + k) * H + h) * (int64_t)kP + p) * NS + 16 * nt_own + 4 * lg;
      if (TAPS && a.tap_s8) *(uint32_t*)(a.tap_s8 + so) = pack_pairs(S8a[j], S8b[j]);
      if (TAPS && a.tap_passed) *(uint32_t*)(a.tap_passed + so) = H8[j];
    }
#pragma unroll
    for (int q = 0; q < KN; ++q) qc2[1][q] = qcn1[q];
    qd_cur = qd_next;
  }
  // the last (redundant) loads land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (a.final_state) {
    const int l16 = tid0 & 15, lg = (tid0 & (kWave - 1)) >> 4;
#pragma unroll
    for (int j = 0; j < PTW; ++j) {
      const int p = 16 * (pt0 + j) + l16;
      const int64_t fo = ((b * H + h) * (int64_t)kP + p) * NS + 16 * nt_own + 4 * lg;
      *(uint32_t*)(a.final_state + fo) = H8[j];
    }
  }
}

// One launch for both parts: whole heads in blocks [0, nfull), then the p
// halves of the partial last round, which start on each CU as soon as its last
// whole head is done. The LDS arrays are declared once here, as separate
// objects (the compiler then knows the Q(B) copy target aliases none of the
// other arrays).
template <int DT, int LC, int NS, bool TAPS>
__global__ __launch_bounds__(kThreadsI8, 1) void k_fused_i8(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) u16 s_xT[2 * kP * (LC + kXTPad)];
  __shared__ __attribute__((aligned(16))) int8_t s_qB[LC * NS];
  __shared__ __attribute__((aligned(16))) int8_t s_qx[2 * kP * LC];
  __shared__ __attribute__((aligned(16))) int8_t s_h8[kP * NS];
  __shared__ __attribute__((aligned(16))) float s_vec[2 * 2 * LC];
  __shared__ __attribute__((aligned(16))) float s_vw[kWaves * LC];
  __shared__ __attribute__((aligned(16))) float s_ss[3 * kP];
  const int64_t bid = blockIdx.x;
  if (bid < a.nfull)
    fused_i8_body<DT, LC, NS, 4, TAPS>(a, bid, s_xT, s_qB, s_qx, s_h8, s_vec, s_vw, s_ss);
  else
    fused_i8_body<DT, LC, NS, 2, TAPS>(a, bid - a.nfull, s_xT, s_qB, s_qx, s_h8, s_vec, s_vw, s_ss);
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
  int64_t nfull;  // launch layout as in FusedArgs
  int unit_map;
  int half_il;
};

// LDS arrays of the float kernel, declared once per kernel (see k_fused_i8)
template <int DT, int LC, int NS>
struct FLds {
  static constexpr bool SPLIT = DT == DT_BF16;
  u16* xT;    // x^T (xT_pair layout)
  u16* xs;    // 16-bit (LUT x)^T [p][s] (h_off<LC>); with bf16 the LUT goes on the B side
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
  const auto stage_load = [&](int kc, int tid, Pf& pf) {
    const int t0 = kc * LC;
    const int lim = min(LC - 1, (int)d.L - 1 - t0);
    const int it = tid % XI;
    const int q = it / C8N, c8 = c8b + it % C8N;
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
      const int q = tid / C8N, c8 = c8b + tid % C8N;
      const uint32_t* w0 = (const uint32_t*)&xr[0];
      const uint32_t* w1 = (const uint32_t*)&xr[1];
      const uint32_t* w2 = (const uint32_t*)&xr[2];
      const uint32_t* w3 = (const uint32_t*)&xr[3];
      u16* const xTb = s_xT + xT_pair<LC>(8 * c8, q >> 3, q & 3) + 4 * ((q >> 2) & 1);  // as in the INT8 kernel
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *(uint2*)(xTb + (2 * e) * (LC + kXTPad)) =
            make_uint2(__builtin_amdgcn_perm(w1[e], w0[e], 0x05040100u), __builtin_amdgcn_perm(w3[e], w2[e], 0x05040100u));
        *(uint2*)(xTb + (2 * e + 1) * (LC + kXTPad)) =
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
          *(uint2*)&s_xs[h_off<LC>(8 * c8 + e, 4 * q)] = make_uint2(pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3]));
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
  // C rows (B operand over N) of this wave's row tiles {w, 15 - w}
  // C rows of row tile {w, 15 - w}[rr] of chunk kc
  const auto load_C = [&](int kc, int lane, int rr, uint4 (&cf)[KNF]) {
    const int t0 = kc * LC;
    const int lim = min(LC - 1, (int)d.L - 1 - t0);
    const int l16 = lane & 15, lg = lane >> 4;
    const T* c0 = Cb + (int64_t)t0 * rowB;
    const int i = min((rr == 0) ? w : 2 * kWaves - 1 - w, RT - 1);
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
        for (int j = 0; j < PTW; ++j) b_[j] = frag16<DT>(&s_xs[h_off<LC>(16 * (pt0 + j) + l16, s0)]);
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
      const int i = (rr == 0) ? w : 2 * kWaves - 1 - w;
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
  __shared__ __attribute__((aligned(16))) u16 s_xT[kP * (LC + kXTPad)];
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
  const Dims& d = fa.d;
  const int64_t BH = d.B * d.H;
  const int64_t ncu = cu_count();
  int64_t nhalf = 0;
  if (ncu > 0) {
    const int64_t rem = BH % ncu;
    if (rem != 0 && 2 * rem <= ncu) nhalf = rem;
  }
  const int64_t nfull = BH - nhalf;
  return K::launch(fa, nfull, nhalf, (d.B * d.G) % 8 == 0, nfull % 8 == 0 && nhalf % 8 == 0, st);
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

template <int DT, int LC, int NS>
struct Int8Launch {
  static hipError_t launch(FusedArgs fa, int64_t nfull, int64_t nhalf, bool unit_map, bool half_il,
                           hipStream_t st) {
    fa.nfull = nfull;
    fa.unit_map = unit_map;
    fa.half_il = half_il;
    const int64_t blocks = nfull + 2 * nhalf;
    if (blocks == 0) return hipSuccess;
    if (fa.tap_qxs || fa.tap_s32 || fa.tap_s8 || fa.tap_passed)
      hipLaunchKernelGGL((k_fused_i8<DT, LC, NS, true>), dim3((unsigned)blocks), dim3(kThreadsI8), 0, st, fa);
    else
      hipLaunchKernelGGL((k_fused_i8<DT, LC, NS, false>), dim3((unsigned)blocks), dim3(kThreadsI8), 0, st, fa);
    return hipGetLastError();
  }
};

template <int DT, int LC, int NS>
hipError_t launch_main(const FusedArgs& fa, hipStream_t st) {
  return launch_split<Int8Launch<DT, LC, NS>>(fa, st);
}

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
  if (!int8) return 2 * al((size_t)d.B * d.H * d.c * d.l * sizeof(float));
  const size_t Lp = (size_t)d.c * d.l;
  const size_t qbc = (size_t)d.B * Lp * d.G * d.N;
  const size_t cs = (size_t)d.B * d.H * d.c * d.l * sizeof(float);
  const size_t qd = (size_t)d.B * d.H * d.c;
  return 2 * al(qbc) + 2 * al(cs) + al(qd);
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
  const size_t Lp = (size_t)d.c * d.l;
  const size_t qbc = (size_t)d.B * Lp * d.G * d.N;
  const size_t cs = (size_t)d.B * d.H * d.c * d.l * sizeof(float);
  char* w = (char*)ws;
  int8_t* qB = (int8_t*)w;
  w += al(qbc);
  int8_t* qC = (int8_t*)w;
  w += al(qbc);
  float* dAcs = (float*)w;
  w += al(cs);
  float* lut = (float*)w;
  w += al(cs);
  uint8_t* qd = (uint8_t*)w;

  // ChunkCumsum and the B/C prologue in one launch when the block count allows
  const int64_t ncs = (int64_t)d.c * d.B * ((d.H + kCsHeads - 1) / kCsHeads);
  const int64_t npro = (int64_t)d.c * (d.l / kPrepRows) * d.B * d.G;
  hipError_t e;
  if (ncs + npro < ((int64_t)1 << 24) && d.B <= 65535) {
    const dim3 grid((unsigned)(ncs + npro));
    if (dtype == DT_F16)
      hipLaunchKernelGGL(k_prep_i8<DT_F16>, grid, dim3(kCsThreads), 0, st, d, dt, A, dAcs, lut, qd, B, C,
                         sc.inv_B, sc.inv_C, qB, qC, (int)ncs);
    else
      hipLaunchKernelGGL(k_prep_i8<DT_BF16>, grid, dim3(kCsThreads), 0, st, d, dt, A, dAcs, lut, qd, B, C,
                         sc.inv_B, sc.inv_C, qB, qC, (int)ncs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    const dim3 pgrid((unsigned)(d.c * (d.l / 64)), (unsigned)(d.B * d.G));
    if (dtype == DT_F16)
      hipLaunchKernelGGL(k_prologue_bc<DT_F16>, pgrid, dim3(256), 0, st, d, B, C, sc.inv_B, sc.inv_C, qB, qC);
    else
      hipLaunchKernelGGL(k_prologue_bc<DT_BF16>, pgrid, dim3(256), 0, st, d, B, C, sc.inv_B, sc.inv_C, qB, qC);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_chunk_cumsum(d, dtype, dt, A, dAcs, lut, qd, st);
    if (e != hipSuccess) return e;
  }

  const FusedArgs fa{d, X, dt, qB, qC, dAcs, lut, qd, D, sc, Y, (const int8_t*)initial_state,
                     (int8_t*)final_state, tap_qxs, tap_s32, tap_s8, tap_passed, 0, 0, 0};
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
