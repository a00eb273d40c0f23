// Device helpers shared by the gfx950 kernels of the EAGLE draft-and-verify path.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/eagle.h"

namespace eagle {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16s;   // bf16 storage (bit pattern)

constexpr int kSlots = EAGLE_MAX_SLOTS;
constexpr int kMaxPos = EAGLE_MAX_POSITIONS;
constexpr int kMaxTopK = EAGLE_MAX_TOPK;

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16, round to nearest even (inf/nan kept)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Storage-type traits.  A "vector" is 16 bytes: VEC elements.  One vector per
// lane feeds one 16x16 MFMA step whose K-extent is 4*VEC (bf16: one
// v_mfma_f32_16x16x32_bf16; fp32: four v_mfma_f32_16x16x4_f32).  Lane l holds
// row/column (l & 15) and K-group (l >> 4) of the operands; the accumulator
// holds rows 4*(l>>4) + 0..3 of column (l & 15).
template <typename T> struct DT;

template <> struct DT<bf16s> {
  static constexpr int VEC = 8;
  __device__ static __forceinline__ float ld(const bf16s* p) { return bf2f(*p); }
  __device__ static __forceinline__ void st(bf16s* p, float v) { *p = (bf16s)f2bf(v); }
  __device__ static __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ float elem(const u32x4& v, int e) {
    uint32_t w = v[e >> 1];
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
  // pack VEC floats into a vector
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = f2bf(f[2 * i]) | (f2bf(f[2 * i + 1]) << 16);
    return r;
  }
};

template <> struct DT<float> {
  static constexpr int VEC = 4;
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void st(float* p, float v) { *p = v; }
  __device__ static __forceinline__ f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
    return c;
  }
  __device__ static __forceinline__ float elem(const u32x4& v, int e) { return __uint_as_float(v[e]); }
  __device__ static __forceinline__ u32x4 pack(const float* f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(f[i]);
    return r;
  }
};

// One row of an activation source: base + (idx ? idx[m] : m) * stride elements.
// Gathered indices are clamped to [0, limit) when limit > 0 (token ids index
// the embedding table; a bad id must not read outside it).
struct RowSrc {
  const void* base;
  const int32_t* idx;
  int64_t stride;
  int64_t limit;
};

template <typename T>
__device__ __forceinline__ const T* row_ptr(const RowSrc& s, int m) {
  int64_t r = s.idx ? (int64_t)s.idx[m] : (int64_t)m;
  if (s.limit > 0) r = r < 0 ? 0 : (r >= s.limit ? s.limit - 1 : r);
  return reinterpret_cast<const T*>(s.base) + r * s.stride;
}

// wave64 reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// s_waitcnt immediate for vmcnt(n) alone (vmcnt bits [3:0] and [15:14])
constexpr int vm_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
// LDS pointers for the direct-to-LDS loads and the transposing LDS reads
typedef __attribute__((address_space(3))) void lds_void;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

// Wave reductions without LDS permutes: a DPP butterfly inside each 16-lane
// row (quad pairs, quad swap, half-row mirror, row mirror) leaves every lane
// of a row with the row's result, then four lane reads combine the rows.  The
// result is wave-uniform.  Every lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float rows_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float rows_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) +
         (readlane_f(v, 32) + readlane_f(v, 48));
}
// float -> unsigned with the same order (-0 taken as +0, NaN below everything)
__device__ __forceinline__ uint32_t float_order(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  const uint32_t o = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return x != x ? 0u : o;
}
__device__ __forceinline__ float order_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t rows_umax64(uint64_t v) {
  v = umax64(v, dpp_u64<0xB1>(v));
  v = umax64(v, dpp_u64<0x4E>(v));
  v = umax64(v, dpp_u64<0x141>(v));
  v = umax64(v, dpp_u64<0x140>(v));
  return umax64(umax64(readlane_u64(v, 0), readlane_u64(v, 16)), umax64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// Exchanges across 16-lane rows as VALU swaps (v_permlane16_swap /
// v_permlane32_swap): with both operands v, the two results hold, per lane,
// v and the value of lane l ^ 16 (resp. l ^ 32), so a max or a sum of the pair
// equals the xor-shuffle reduction bit for bit (both are commutative).
__device__ __forceinline__ float max_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// (value desc, id asc) ordering used by every top-k / argmax
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ void wave_best(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(i, o, 64);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

}  // namespace eagle
