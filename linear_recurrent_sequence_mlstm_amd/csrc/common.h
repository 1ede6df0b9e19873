// Device helpers shared by the mLSTM / retention kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlstm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// log(sigmoid(x)) = min(x, 0) - log1p(exp(-|x|)), in log2 units.  log1p is
// taken as log2(u) * e / (u - 1) with u = 1 + e (exact for e = 0 up to the
// rounding of u; Goldberg's compensation), so hardware log2/exp2 suffice.
__device__ __forceinline__ float log2_sigmoid(float x) {
  const float e = exp2_fast(-fabsf(x) * kLog2e);  // e^{-|x|} in (0, 1]
  const float u = 1.f + e;
  const float d = u - 1.f;
  const float l = d == 0.f ? e * kLog2e : __builtin_amdgcn_logf(u) * (e * __builtin_amdgcn_rcpf(d));
  return fminf(x, 0.f) * kLog2e - l;
}

__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// MFMA traits: one 16x16 output tile, K elements of the contraction per
// instruction, KL of them held by each lane.  Lane l holds A[l%16][KL*(l/16)+e],
// B[KL*(l/16)+e][l%16] and D[4*(l/16)+i][l%16].
template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  static constexpr int K = 32;
  static constexpr int KL = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const __bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ __forceinline__ static frag zero() {
    frag z;
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
    return z;
  }
  __device__ __forceinline__ static frag ones() {
    frag z;
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)1.f;
    return z;
  }
};

template <>
struct Mma<float> {
  static constexpr int K = 4;
  static constexpr int KL = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
  __device__ __forceinline__ static frag zero() { return 0.f; }
  __device__ __forceinline__ static frag ones() { return 1.f; }
};

// Sum over the four 16-lane groups of a wave, valid in lanes 0..15 (gfx950
// lane swaps: lanes 32..63 meet lanes 0..31, then lanes 16..31 meet 0..15).
__device__ __forceinline__ float sum_lane_groups(float x) {
  const unsigned u = __float_as_uint(x);
  const float s = x + __uint_as_float(__builtin_amdgcn_permlane32_swap(u, u, false, false)[1]);
  const unsigned v = __float_as_uint(s);
  return s + __uint_as_float(__builtin_amdgcn_permlane16_swap(v, v, false, false)[1]);
}

// Vector of 16 bytes of element type T.
template <typename T>
struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  T v[N];
};

template <typename T>
__device__ __forceinline__ Vec16<T> load16(const T* p) {
  Vec16<T> r;
  *reinterpret_cast<uint4*>(r.v) = *reinterpret_cast<const uint4*>(p);
  return r;
}

template <typename T>
__device__ __forceinline__ Vec16<T> zero16() {
  Vec16<T> r;
  *reinterpret_cast<uint4*>(r.v) = make_uint4(0, 0, 0, 0);
  return r;
}

// Buffer resource over [base, base + bytes): loads past the end return zero,
// so masked (ragged-tail) loads need no branch.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Callers pass wave-uniform values; readfirstlane states that, so the
// descriptor lives in scalar registers (a descriptor the compiler believes
// divergent is used through a waterfall loop around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  void* ub = reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

template <typename T>
__device__ __forceinline__ Vec16<T> bload16(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  Vec16<T> v;
  *reinterpret_cast<u32x4*>(v.v) = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return v;
}

// one element (bf16 or fp32) as float
template <typename T>
__device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, unsigned byte_off);
template <>
__device__ __forceinline__ float bload1<float>(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}
template <>
__device__ __forceinline__ float bload1<__bf16>(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0) << 16);
}

// one element, raw bits (no conversion, so that the load need not complete
// until the value is used)
template <typename T>
__device__ __forceinline__ unsigned bload1_raw(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  if constexpr (sizeof(T) == 2) return (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}
template <typename T>
__device__ __forceinline__ float raw_to_f32(unsigned x) {
  return __uint_as_float(sizeof(T) == 2 ? x << 16 : x);
}

// four consecutive elements as floats
template <typename T>
__device__ __forceinline__ void bload4(__amdgpu_buffer_rsrc_t r, unsigned byte_off, float (&x)[4]);
template <>
__device__ __forceinline__ void bload4<float>(__amdgpu_buffer_rsrc_t r, unsigned byte_off, float (&x)[4]) {
  const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(u[i]);
}
template <>
__device__ __forceinline__ void bload4<__bf16>(__amdgpu_buffer_rsrc_t r, unsigned byte_off, float (&x)[4]) {
  const u32x2 u = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
  x[0] = __uint_as_float(u[0] << 16);
  x[1] = __uint_as_float(u[0] & 0xffff0000u);
  x[2] = __uint_as_float(u[1] << 16);
  x[3] = __uint_as_float(u[1] & 0xffff0000u);
}

// Four consecutive elements, raw bits (converted where used, so that the
// load need not complete before then).
template <typename T>
struct Raw4;
template <>
struct Raw4<__bf16> {
  u32x2 v;
};
template <>
struct Raw4<float> {
  u32x4 v;
};
template <typename T>
__device__ __forceinline__ Raw4<T> bload4_raw(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  Raw4<T> x;
  if constexpr (sizeof(T) == 2) x.v = __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
  else x.v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return x;
}
template <typename T>
__device__ __forceinline__ void raw4_to_f32(const Raw4<T>& r, float (&x)[4]) {
  if constexpr (sizeof(T) == 2) {
    x[0] = __uint_as_float(r.v[0] << 16);
    x[1] = __uint_as_float(r.v[0] & 0xffff0000u);
    x[2] = __uint_as_float(r.v[1] << 16);
    x[3] = __uint_as_float(r.v[1] & 0xffff0000u);
  } else {
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(r.v[i]);
  }
}
// One element converted to T and stored through a buffer resource (a store
// past its end is dropped).
template <typename T>
__device__ __forceinline__ void bstore1(__amdgpu_buffer_rsrc_t r, unsigned byte_off, float a) {
  if constexpr (sizeof(T) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)a), r, byte_off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r, byte_off, 0, 0);
}
// Four consecutive elements converted to T and stored through a buffer
// resource (stores past its end are dropped).
template <typename T>
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, unsigned byte_off, float a, float b, float c,
                                        float d) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    v[2] = (__bf16)c;
    v[3] = (__bf16)d;
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, byte_off, 0, 0);
  } else {
    u32x4 v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 0);
  }
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, output lane i holds element (i & 3) of the 4 elements that source lane
// 4e + (i >> 2) addressed, for e = 0..3.  So if source lane s addresses row
// r0 + (s >> 2), column c0 + 4 (s & 3) of a row-major tile, output lane i
// receives column c0 + i of rows r0 .. r0+3: an MFMA fragment along the rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 ds_read_tr16(const __bf16* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<__bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// Direct global-to-LDS load of 16 bytes per lane (gfx950 buffer_load_dwordx4
// ... lds): lane l writes bytes [lds + 16 l, lds + 16 l + 16) of the wave-uniform
// LDS address lds, read from voff + soff of the buffer (zero past its end).
// It completes under vmcnt like any buffer load.  Kept in a device function:
// the address-space cast must not appear in a kernel body that the host pass
// also sees.
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds, unsigned voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Two floats to a packed pair of bf16 (first one in the low half): one
// v_cvt_pk_bf16_f32, where element-wise conversions would also need a permute.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Four consecutive elements to an 8- (bf16) or 16-byte (fp32) aligned address.
__device__ __forceinline__ void store4(__bf16* dst, __bf16 a, __bf16 b, __bf16 c, __bf16 d) {
  bf16x4 v;
  v[0] = a;
  v[1] = b;
  v[2] = c;
  v[3] = d;
  *reinterpret_cast<bf16x4*>(dst) = v;
}
__device__ __forceinline__ void store4(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}
// Four floats rounded to T, stored as in store4 (bf16: two packed converts).
__device__ __forceinline__ void store4f(__bf16* dst, float a, float b, float c, float d) {
  const u32x2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<u32x2*>(dst) = v;
}
__device__ __forceinline__ void store4f(float* dst, float a, float b, float c, float d) { store4(dst, a, b, c, d); }

}  // namespace mlstm
