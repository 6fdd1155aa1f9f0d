// Data layouts shared by the fused INT8 kernels: the operand fragments the
// preparation launch writes (Q(B)^T for ChunkState, CB' for ChunkScan2), the
// LDS tiles and their swizzles, and the gfx950 transposing LDS reads.
#pragma once

#include "ssd_device.hpp"

namespace ssd {

constexpr int kHP = 64;                         // head dim covered (P)
constexpr float kLn2Inv = 1.4426950408889634f;  // log2(e)

// ChunkScan exponent vectors of one position s of a chunk: A_s = a_s log2(e)
// and B_s = A_s - log2(dt_s) + E, so that exp2(A_r - B_s) = exp(a_r - a_s)
// dt_s 2^-E (dt = 0 past L gives B = +inf and weight 0). Each operation is
// rounded on its own (no contraction into an FMA), so every kernel that builds
// the vectors gets the same bits and the schedules give the same Y.
__device__ __forceinline__ void scan_vectors(float a_s, float dt_s, float E, float& A, float& B) {
#pragma clang fp contract(off)
  A = a_s * kLn2Inv;
  B = (A - __builtin_amdgcn_logf(dt_s)) + E;
}

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef unsigned u2v_t __attribute__((ext_vector_type(2)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef short v8s_t __attribute__((ext_vector_type(8)));

// ChunkScan2 operand fragments per (batch, chunk, group): row tile i (16
// positions s) pairs with column tiles (2m, 2m + 1), m = 0 .. i / 2.
__host__ __device__ constexpr int cb_frags(int lc) {
  int n = 0;
  for (int i = 0; i < lc / 16; ++i) n += i / 2 + 1;
  return n;
}
__host__ __device__ constexpr int cb_frag_base(int i) {  // sum over i' < i of (i' / 2 + 1)
  return (i & 1) ? ((i + 1) / 2) * ((i + 1) / 2) : (i / 2) * (i / 2 + 1);
}

// The power of two E of the CB' fragments of a group: t = N 127^2 s_C s_B bounds
// |CB s_C s_B|; with t = f 2^e, f in [0.5, 1), |CB s_C s_B 2^(15 - e)| < 2^15.
__device__ __forceinline__ int cb_exp(float scb, int N) {
  const float t = scb * (float)(N * 16129);
  const int e = (int)((__float_as_uint(t) >> 23) & 0xff) - 126;
  return min(max(15 - e, -100), 100);
}

// Transposing LDS reads. 8-bit: the 16 lanes of a group each point at 8 bytes;
// lanes 2r, 2r + 1 form row r (16 bytes) of an 8 x 16 byte matrix and lane i
// receives column i (byte i of rows 0..7). 16-bit: lanes 4r .. 4r + 3 form row r
// (16 elements) of a 4 x 16 matrix and lane i receives element i of rows 0..3.
__device__ __forceinline__ v2i_t ldtr8(const int8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i_t*)(int8_t*)p);
}
__device__ __forceinline__ v4s_t ldtr16(const u16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(u16*)p);
}

// byte tiles [rows][W]: 16-byte chunks XOR-swizzled with the low row bits
template <int W>
__device__ __forceinline__ int bsw(int r, int c) {
  constexpr int nch = W / 16;
  return r * W + 16 * ((c >> 4) ^ (r & (nch - 1) & 7)) + (c & 15);
}

// x tile [s][64] (2-byte elements, rows of 128 bytes): the 16-byte chunk index
// is XORed with 2 ((s ^ (s >> 2)) & 3). The transposing reads of a ChunkScan2
// operand (16 consecutive rows, 32 bytes each) and the producers' row writes
// are then free of bank conflicts, and the swizzle of row s = 32 m + 16 h +
// 4 g + r is 2 (g ^ r), the same for every m and h.
__device__ __forceinline__ int xsw_off(int s, int p) {  // element offset; p multiple of 4
  return s * kHP + 8 * ((p >> 3) ^ (2 * ((s ^ (s >> 2)) & 3))) + (p & 7);
}
// Q(X_scaled) tile [s][64] (bytes): chunk index XOR ((s >> 1) & 3) ^ ((s >> 4) & 3);
// for the ChunkState reads (rows s = 64 ks + 16 g + 8 h + r) that is (r >> 1) ^ g.
__device__ __forceinline__ int qsw_off(int s, int p) {  // byte offset; p multiple of 8
  return s * kHP + 16 * ((p >> 4) ^ (((s >> 1) & 3) ^ ((s >> 4) & 3))) + (p & 15);
}
// Position order of the per-position tables that ChunkScan2 reads by K slot:
// s' = 32 m + 16 h + 4 g + r sits at 32 m + 8 g + 4 h + r, so lane group g reads
// its eight K values (h = 0, 1; r = 0..3) as 32 contiguous bytes.
__device__ __forceinline__ int kperm(int s) {
  return (s & ~31) + 8 * ((s >> 2) & 3) + 4 * ((s >> 4) & 1) + (s & 3);
}


// Four consecutive scale values (the scale arrays are only 4-byte aligned).
__device__ __forceinline__ float4 ld_scale4(const float* p) { return make_float4(p[0], p[1], p[2], p[3]); }

}  // namespace ssd
