// Shared device helpers and host-side validation for libkvmem (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <string>

#include "kvm.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

namespace kvm {

// ------------------------------------------------------------------------------ host side

kvm_status set_error(kvm_status s, const char* fmt, ...);
kvm_status check_hip(hipError_t e, const char* what);
kvm_status require_gfx950();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define KVM_REQUIRE(cond, status, ...)                 \
  do {                                                 \
    if (!(cond)) return ::kvm::set_error(status, __VA_ARGS__); \
  } while (0)

#define KVM_PTR(p) KVM_REQUIRE((p) != nullptr, KVM_ERR_NULL, "%s is NULL", #p)
#define KVM_ALIGNED(p) KVM_REQUIRE(::kvm::aligned16(p), KVM_ERR_ALIGN, "%s is not 16-byte aligned", #p)
#define KVM_PTR_ALIGNED(p) do { KVM_PTR(p); KVM_ALIGNED(p); } while (0)
#define KVM_OPT_ALIGNED(p) do { if (p) KVM_ALIGNED(p); } while (0)

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------------------------ device side

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Load EPL consecutive elements (16 bytes) as floats.
template <typename T> struct Vec16;
template <> struct Vec16<uint16_t> {  // bf16 storage
  static constexpr int N = 8;
  __device__ __forceinline__ static void load(const uint16_t* p, float (&out)[8]) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  }
  __device__ __forceinline__ static void unpack(const uint4& v, float (&out)[8]) {
    out[0] = bf16_lo(v.x); out[1] = bf16_hi(v.x);
    out[2] = bf16_lo(v.y); out[3] = bf16_hi(v.y);
    out[4] = bf16_lo(v.z); out[5] = bf16_hi(v.z);
    out[6] = bf16_lo(v.w); out[7] = bf16_hi(v.w);
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float (&out)[4]) {
    float4 v = *reinterpret_cast<const float4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  __device__ __forceinline__ static void unpack(const uint4& v, float (&out)[4]) {
    out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  }
};

template <typename T> __device__ __forceinline__ float load_scalar(const T* p);
template <> __device__ __forceinline__ float load_scalar<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <> __device__ __forceinline__ float load_scalar<float>(const float* p) { return *p; }

// Cross-lane sums inside groups of N consecutive lanes (N in 1..64); every lane of the group
// ends with the group total.
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float swz_xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}
__device__ __forceinline__ float shfl_xor32(float x) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __float_as_int(x)));
}

template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
  if (N >= 2) x += dpp<0xB1>(x);        // xor 1
  if (N >= 4) x += dpp<0x4E>(x);        // xor 2
  if (N == 8) x += dpp<0x141>(x);       // mirror within 8 lanes
  if (N >= 16) { x += dpp<0x124>(x); x += dpp<0x128>(x); }   // rotate 4, 8 within 16
  if (N >= 32) x += swz_xor16(x);
  if (N >= 64) x += shfl_xor32(x);
  return x;
}
template <int N> __device__ __forceinline__ float group_max(float x) {
  if (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
  if (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
  if (N == 8) x = fmaxf(x, dpp<0x141>(x));
  if (N >= 16) { x = fmaxf(x, dpp<0x124>(x)); x = fmaxf(x, dpp<0x128>(x)); }
  if (N >= 32) x = fmaxf(x, swz_xor16(x));
  if (N >= 64) x = fmaxf(x, shfl_xor32(x));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

// Order-preserving u32 key of a score (ascending with the value): NaN orders as -inf and
// -0 as +0, so equal keys mean equal scores.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) u = 0xff800000u;  // NaN -> -inf
  if (u == 0x80000000u) u = 0u;                           // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Buffer resource over `bytes` bytes from `base`: loads at offsets past the end return zeros
// without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// LDS tiles whose rows are P 16-byte pieces (P = 16: 128 bf16; P = 8: 64 bf16): piece q of
// row r is stored at position q ^ piece_swz<P>(r).  Sixteen consecutive rows reading the same
// piece then hit sixteen different 16-byte bank groups, so 16-byte operand reads down a
// column meet no bank conflicts.
template <int P>
__device__ __forceinline__ int piece_swz(int r) {
  static_assert(P == 8 || P == 16, "pieces per row");
  return P == 16 ? (r & 15) : ((r >> 1) & 7);
}

// x = h + m + l in bf16 (round to nearest even at each step; ~24 bits of x), 8 values with
// the packed hardware conversion
__device__ __forceinline__ void split3_bf16x8(const float (&x)[8], bf16x8_t& h, bf16x8_t& m, bf16x8_t& l) {
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const f32x2_t v = {x[j], x[j + 1]};
    const bf16x2_t hh = __builtin_convertvector(v, bf16x2_t);
    const f32x2_t r1 = {v[0] - (float)hh[0], v[1] - (float)hh[1]};
    const bf16x2_t mm = __builtin_convertvector(r1, bf16x2_t);
    const f32x2_t r2 = {r1[0] - (float)mm[0], r1[1] - (float)mm[1]};
    const bf16x2_t ll = __builtin_convertvector(r2, bf16x2_t);
    h[j] = hh[0]; h[j + 1] = hh[1];
    m[j] = mm[0]; m[j + 1] = mm[1];
    l[j] = ll[0]; l[j + 1] = ll[1];
  }
}

// 16 bytes at byte offset `off` of a buffer (zeros past its end)
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, int off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float phi_f(float x) { return x > 0.f ? x + 1.f : __expf(x); }
__device__ __forceinline__ float sigmoid_f(float x) {
  float e = __expf(-fabsf(x));
  return x >= 0.f ? 1.f / (1.f + e) : e / (1.f + e);
}

}  // namespace kvm
