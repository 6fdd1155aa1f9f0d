// Device-side helpers shared by the SSD kernels (gfx950 / CDNA4, wave64).
//
// MFMA fragments used throughout (16x16 output tiles, wave64):
//   A operand: lane L carries row (L % 16) and a group of consecutive K values
//              selected by L / 16;
//   B operand: lane L carries column (L % 16) and the same K group;
//   C/D:       lane L holds rows 4*(L/16) + r, r = 0..3, of column L % 16.
// The K order inside a group only has to agree between A and B, which every
// loader here guarantees by building both from the same (L/16, e) -> k map.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint16_t u16;

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// storage <-> fp32 conversion
// ---------------------------------------------------------------------------
template <int DT>
struct Store;
template <>
struct Store<DT_F32> {
  typedef float T;
  static __device__ __forceinline__ float to_f(T v) { return v; }
  static __device__ __forceinline__ T from_f(float v) { return v; }
};
template <>
struct Store<DT_F16> {
  typedef _Float16 T;
  static __device__ __forceinline__ float to_f(T v) { return (float)v; }
  static __device__ __forceinline__ T from_f(float v) { return (_Float16)v; }
};
template <>
struct Store<DT_BF16> {
  typedef u16 T;  // bf16 bit pattern
  static __device__ __forceinline__ float to_f(T v) { return __uint_as_float(((uint32_t)v) << 16); }
  static __device__ __forceinline__ T from_f(float v) {
    return __builtin_bit_cast(u16, (__bf16)v);  // round to nearest even
  }
};

// Two values rounded (to nearest even) to the 16-bit type, packed low/high in
// one dword (one packed conversion instruction).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  static_assert(DT == DT_F16 || DT == DT_BF16, "16-bit types only");
  if constexpr (DT == DT_F16) {
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const h2_t v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    const b2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

template <int DT>
__device__ __forceinline__ float ld_f(const void* p, int64_t i) {
  return Store<DT>::to_f(((const typename Store<DT>::T*)p)[i]);
}

// Load 8 consecutive elements (16-byte aligned for 2-byte types, 32-byte for fp32).
template <int DT>
__device__ __forceinline__ void ld8_f(const void* p, int64_t i, float out[8]) {
  if constexpr (DT == DT_F32) {
    const float4* q = (const float4*)((const float*)p + i);
    float4 a = q[0], b = q[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  } else {
    uint4 v = *(const uint4*)((const u16*)p + i);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (DT == DT_F16) {
        out[2 * j] = (float)__builtin_bit_cast(_Float16, (u16)(w[j] & 0xffff));
        out[2 * j + 1] = (float)__builtin_bit_cast(_Float16, (u16)(w[j] >> 16));
      } else {
        out[2 * j] = __uint_as_float(w[j] << 16);
        out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// quantiser arithmetic (single fp32 roundings, round half away from zero)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int q_sat(float v, float qmax) {
  // roundf is round-half-away-from-zero; the clamp saturates to +-qmax.
  return (int)fminf(fmaxf(roundf(v), -qmax), qmax);
}

// int8 x 4 packing
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)d << 24);
}
__device__ __forceinline__ int byte_s(uint32_t w, int j) { return (int)(int8_t)(w >> (8 * j)); }

// Rounding shift of Eq. 6: sign(v) * ((|v| + 64) >> 7).
__device__ __forceinline__ int rsh7(int v) {
  int m = (v < 0 ? -v : v);
  int r = (m + 64) >> 7;
  return v < 0 ? -r : r;
}

// Saturating int8 quantiser with round half away from zero. After the clamp,
// trunc(c + copysign(0.5 - 2^-25, c)) equals RHAZ(c) for every float32 c
// (checked exhaustively over all 2^32 bit patterns in the test-suite).
__device__ __forceinline__ float q8_pre(float v) {
  const float c = fminf(fmaxf(v, -127.f), 127.f);
  return c + __builtin_copysignf(0.49999997f, c);
}
__device__ __forceinline__ int q8(float v) { return (int)q8_pre(v); }

// Four such codes packed into one dword (byte j from v_j). The float -> int
// conversion writes its low byte straight into the destination byte (SDWA
// dst_sel), so the packing costs no extra instructions.
__device__ __forceinline__ uint32_t q8x4(float v0, float v1, float v2, float v3) {
  uint32_t d = (uint32_t)q8(v0);
  asm("v_cvt_i32_f32_sdwa %0, %1 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
      : "+v"(d) : "v"(q8_pre(v1)));
  asm("v_cvt_i32_f32_sdwa %0, %1 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
      : "+v"(d) : "v"(q8_pre(v2)));
  asm("v_cvt_i32_f32_sdwa %0, %1 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
      : "+v"(d) : "v"(q8_pre(v3)));
  return d;
}

// Eq. 6 rounding shift sign(v) * ((|v| + 64) >> 7) in arithmetic-shift form:
// (v + 64 + (v >> 31)) >> 7 (equal for every |v| <= 128 * 127; tested).
__device__ __forceinline__ int rsh7_fast(int v) { return (v + 64 + (v >> 31)) >> 7; }

__device__ __forceinline__ int sat127(int v) { return min(max(v, -127), 127); }

// Packed 16-bit helpers of the Eq. 6 update (two state elements per lane op).
typedef short v2s __attribute__((ext_vector_type(2)));

// Two int8 codes from float values prepared by q8_pre, as int16 halves of one
// dword: the second conversion writes its low 16 bits into the high half.
__device__ __forceinline__ v2s cvt_pair(float c0, float c1) {
  uint32_t d = (uint32_t)(int)c0;
  asm("v_cvt_i32_f32_sdwa %0, %1 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD"
      : "+v"(d) : "v"(c1));
  return __builtin_bit_cast(v2s, d);
}

// Two signed bytes of w (picked by the permute selector into bits 15:8 and
// 31:24) as sign-extended int16 halves.
__device__ __forceinline__ v2s unpack_pair(uint32_t w, uint32_t sel) {
  return __builtin_bit_cast(v2s, __builtin_amdgcn_perm(w, w, sel)) >> (short)8;
}

// RSH7(qd h) = (qd h + 64 + [qd h < 0 ? -1 : 0]) >> 7 per half. qd >= 0, so the
// sign of h stands for the sign of the product (a zero product rounds to 0
// either way); |qd h| <= 128 * 127 fits int16.
__device__ __forceinline__ v2s rsh7_pair(v2s qd, v2s h) {
  return (v2s)(qd * h + (short)64 + (h >> (short)15)) >> (short)7;
}

__device__ __forceinline__ v2s sat127_pair(v2s v) {
  return __builtin_elementwise_min(__builtin_elementwise_max(v, (v2s){-127, -127}), (v2s){127, 127});
}

// Low bytes of the four int16 halves of (lo, hi) as one dword.
__device__ __forceinline__ uint32_t pack_pairs(v2s lo, v2s hi) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo),
                               0x06040200u);
}

// ---------------------------------------------------------------------------
// MFMA wrappers
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4i mma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Compute-type fragment of 8 K values per lane for the floating MFMAs.
template <int DT>
struct FragF;
template <>
struct FragF<DT_F16> {
  v8h v;
  __device__ __forceinline__ void set(int e, float x) { v[e] = (_Float16)x; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (_Float16)0.f;
  }
  static __device__ __forceinline__ v4f mma(const FragF& a, const FragF& b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
  }
};
template <>
struct FragF<DT_BF16> {
  v8bf v;
  __device__ __forceinline__ void set(int e, float x) { v[e] = (__bf16)x; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)0.f;
  }
  static __device__ __forceinline__ v4f mma(const FragF& a, const FragF& b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
  }
};
template <>
struct FragF<DT_F32> {
  float v[8];
  __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  static __device__ __forceinline__ v4f mma(const FragF& a, const FragF& b, v4f c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
  }
};

// Fragment for values computed in the kernel (products such as LUT * x or the
// ChunkScan2 weights), as opposed to exact copies of the inputs. bf16 keeps
// only 8 significant bits, so such a value is carried as hi + lo, two bf16
// numbers, and multiplied with two MFMAs (about 16 significant bits); fp16 and
// fp32 use one plain fragment.
template <int DT>
struct FragC {
  FragF<DT> hi;
  __device__ __forceinline__ void set(int e, float x) { hi.set(e, x); }
  __device__ __forceinline__ void zero() { hi.zero(); }
};
template <>
struct FragC<DT_BF16> {
  FragF<DT_BF16> hi, lo;
  __device__ __forceinline__ void set(int e, float x) {
    const __bf16 h = (__bf16)x;
    hi.v[e] = h;
    lo.v[e] = (__bf16)(x - (float)h);
  }
  __device__ __forceinline__ void zero() {
    hi.zero();
    lo.zero();
  }
};

// acc += a * b with a computed (split) and b an exact input fragment.
template <int DT>
__device__ __forceinline__ v4f mma_ca(const FragC<DT>& a, const FragF<DT>& b, v4f acc) {
  acc = FragF<DT>::mma(a.hi, b, acc);
  if constexpr (DT == DT_BF16) acc = FragF<DT>::mma(a.lo, b, acc);
  return acc;
}
// acc += a * b with a an exact input fragment and b computed (split).
template <int DT>
__device__ __forceinline__ v4f mma_cb(const FragF<DT>& a, const FragC<DT>& b, v4f acc) {
  acc = FragF<DT>::mma(a, b.hi, acc);
  if constexpr (DT == DT_BF16) acc = FragF<DT>::mma(a, b.lo, acc);
  return acc;
}

// Compute-type element stored in LDS for the floating MFMAs.
template <int DT>
struct LdsT {
  typedef typename Store<DT>::T T;
};

template <int DT>
__device__ __forceinline__ typename Store<DT>::T to_store(float x) {
  return Store<DT>::from_f(x);
}

// Read 8 consecutive compute-type values from LDS into a fragment.
template <int DT>
__device__ __forceinline__ void lds_frag8(const typename Store<DT>::T* p, FragF<DT>& f) {
  if constexpr (DT == DT_F16) {
    f.v = *(const v8h*)p;
  } else if constexpr (DT == DT_BF16) {
    f.v = *(const v8bf*)p;
  } else {
    const float4* q = (const float4*)p;
    float4 a = q[0], b = q[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  }
}

// Read 8 consecutive input-dtype values from global memory into a fragment.
template <int DT>
__device__ __forceinline__ void glb_frag8(const void* p, int64_t i, FragF<DT>& f) {
  if constexpr (DT == DT_F16) {
    f.v = *(const v8h*)((const _Float16*)p + i);
  } else if constexpr (DT == DT_BF16) {
    f.v = *(const v8bf*)((const u16*)p + i);
  } else {
    float t[8];
    ld8_f<DT_F32>(p, i, t);
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = t[e];
  }
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
// Wave index within the workgroup, in a scalar register (it is uniform across
// the wave, which lets loops and branches on it stay scalar).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

}  // namespace ssd
