// Device-side helpers for the SketchSSM decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

// Loads of wave-uniform values through the scalar cache: the constant
// address space tells the compiler that the memory does not change while
// the kernel runs (the rank table and decay rates never do; a kernel reads
// each tile's ring fill once, before it writes it), so a uniform address
// becomes an
// s_load, which does not queue behind the vector loads of the waves already
// in flight.
typedef const __attribute__((address_space(4))) int const_int_t;
typedef const __attribute__((address_space(4))) float const_float_t;
__device__ __forceinline__ int uload(const int* base, int i) {
  return ((const_int_t*)base)[i];     // (an address-space cast: C-style)
}
__device__ __forceinline__ float uload(const float* base, int i) {
  return ((const_float_t*)base)[i];
}


constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

typedef uint16_t bf16;  // storage type of bfloat16 values
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float((uint32_t)x << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16)(u >> 16);
}

template <typename T> struct Store;
template <> struct Store<float> {
  static __device__ __forceinline__ float cvt(float x) { return x; }
};
template <> struct Store<bf16> {
  static __device__ __forceinline__ bf16 cvt(float x) { return f32_to_bf16(x); }
};

template <typename T>
__device__ __forceinline__ float ld(const T* p) { return to_f32(*p); }

// Four consecutive elements as fp32.
__device__ __forceinline__ void ld4(const float* p, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void ld4(const bf16* p, float (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(v.x << 16);
  x[1] = __uint_as_float(v.x & 0xffff0000u);
  x[2] = __uint_as_float(v.y << 16);
  x[3] = __uint_as_float(v.y & 0xffff0000u);
}

__device__ __forceinline__ void st4(float* p, const float (&x)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void st4(bf16* p, const float (&x)[4]) {
  uint2 v;
  v.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
  v.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
  *reinterpret_cast<uint2*>(p) = v;
}

template <typename T>
__device__ __forceinline__ void st(T* p, float x) { *p = Store<T>::cvt(x); }

// N consecutive elements (N in {1, 2, 4, 8}) as fp32, with the widest loads
// the alignment of an N-element run allows.
template <int N>
__device__ __forceinline__ void ldn(const float* p, float (&x)[N]) {
  if constexpr (N == 1) {
    x[0] = p[0];
  } else if constexpr (N == 2) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    x[0] = v.x; x[1] = v.y;
  } else {
#pragma unroll
    for (int e = 0; e < N; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + e);
      x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
    }
  }
}
// The state's own stream (read once and written once per tile): N = 2 or 4
// fp32 with the non-temporal cache policy, so that the state passing through
// does not displace the sketch, ring and inputs the other kernels re-read
// from the caches.
template <int N>
__device__ __forceinline__ void ldn_nt(const float* p, float (&x)[N]) {
  static_assert(N == 2 || N == 4, "ldn_nt: 2 or 4 floats");
  typedef float fv __attribute__((ext_vector_type(N)));
  const fv v = __builtin_nontemporal_load(reinterpret_cast<const fv*>(p));
#pragma unroll
  for (int e = 0; e < N; ++e) x[e] = v[e];
}
// 16 bytes with the non-temporal cache policy.
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int N>
__device__ __forceinline__ void stn_nt(float* p, const float (&x)[N]) {
  static_assert(N == 2 || N == 4, "stn_nt: 2 or 4 floats");
  typedef float fv __attribute__((ext_vector_type(N)));
  fv v;
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = x[e];
  __builtin_nontemporal_store(v, reinterpret_cast<fv*>(p));
}

template <int N>
__device__ __forceinline__ void ldn(const bf16* p, float (&x)[N]) {
  if constexpr (N == 1) {
    x[0] = to_f32(p[0]);
  } else if constexpr (N == 2) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    x[0] = __uint_as_float(v << 16); x[1] = __uint_as_float(v & 0xffff0000u);
  } else if constexpr (N == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(v.x << 16); x[1] = __uint_as_float(v.x & 0xffff0000u);
    x[2] = __uint_as_float(v.y << 16); x[3] = __uint_as_float(v.y & 0xffff0000u);
  } else {
#pragma unroll
    for (int e = 0; e < N; e += 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + e);
      x[e] = __uint_as_float(v.x << 16); x[e + 1] = __uint_as_float(v.x & 0xffff0000u);
      x[e + 2] = __uint_as_float(v.y << 16); x[e + 3] = __uint_as_float(v.y & 0xffff0000u);
      x[e + 4] = __uint_as_float(v.z << 16); x[e + 5] = __uint_as_float(v.z & 0xffff0000u);
      x[e + 6] = __uint_as_float(v.w << 16); x[e + 7] = __uint_as_float(v.w & 0xffff0000u);
    }
  }
}

template <int N>
__device__ __forceinline__ void stn(float* p, const float (&x)[N]) {
  if constexpr (N == 1) {
    p[0] = x[0];
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
  } else {
#pragma unroll
    for (int e = 0; e < N; e += 4)
      *reinterpret_cast<float4*>(p + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
  }
}
template <int N>
__device__ __forceinline__ void stn(bf16* p, const float (&x)[N]) {
  if constexpr (N == 1) {
    p[0] = f32_to_bf16(x[0]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
  } else {
#pragma unroll
    for (int e = 0; e < N; e += 4) {
      uint2 v;
      v.x = (uint32_t)f32_to_bf16(x[e]) | ((uint32_t)f32_to_bf16(x[e + 1]) << 16);
      v.y = (uint32_t)f32_to_bf16(x[e + 2]) | ((uint32_t)f32_to_bf16(x[e + 3]) << 16);
      *reinterpret_cast<uint2*>(p + e) = v;
    }
  }
}

// N consecutive elements kept in their storage type (bf16 stays packed two
// per register until used).
template <typename T, int N>
struct alignas(sizeof(T) * N) VecN {
  T v[N];
};
template <int N, typename T>
__device__ __forceinline__ VecN<T, N> ldraw(const T* p) {
  return *reinterpret_cast<const VecN<T, N>*>(p);
}
template <typename T, int N>
__device__ __forceinline__ float vget(const VecN<T, N>& x, int e) { return to_f32(x.v[e]); }

// ldraw with the non-temporal cache policy, for rows a kernel reads once
// (sketch rows, ring entries, state copies): 2, 4, 8 or a multiple of 16
// bytes.
template <int N, typename T>
__device__ __forceinline__ VecN<T, N> ldraw_nt(const T* p) {
  constexpr int B = (int)sizeof(T) * N;
  static_assert(B == 2 || B == 4 || B == 8 || B % 16 == 0, "ldraw_nt: 2, 4, 8 or a multiple of 16 bytes");
  VecN<T, N> r;
  if constexpr (B == 2) {
    const unsigned short v = __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p));
    __builtin_memcpy(&r, &v, 2);
  } else if constexpr (B == 4) {
    const unsigned v = __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p));
    __builtin_memcpy(&r, &v, 4);
  } else if constexpr (B == 8) {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    const u2 v = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
    __builtin_memcpy(&r, &v, 8);
  } else {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int o = 0; o < B; o += 16) {
      const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(reinterpret_cast<const char*>(p) + o));
      __builtin_memcpy(reinterpret_cast<char*>(&r) + o, &v, 16);
    }
  }
  return r;
}

// Raw copy of N consecutive elements (ring appends).
template <int N, typename T>
__device__ __forceinline__ void copyn(T* dst, const T* src) {
  float x[N];
  ldn<N>(src, x);
  stn<N>(dst, x);
}


// Sum of x over the lanes that differ in lane bits [LB, LB+NB); every lane
// receives the total.
template <int LB, int NB>
__device__ __forceinline__ float xsum(float x) {
#pragma unroll
  for (int s = 0; s < NB; ++s) x += __shfl_xor(x, 1 << (LB + s));
  return x;
}

// Reduce a[0..N) across the 2^NB lanes that differ in lane bits
// [LB, LB+NB), halving the vector at every exchange.  Afterwards a lane holds
// in a[0..N>>NB) the sums of elements [sel*(N>>NB), (sel+1)*(N>>NB)) where
// sel = (lane >> LB) & (2^NB - 1).  Requires N >= 2^NB.
template <int N, int LB, int NB>
__device__ __forceinline__ void tr_reduce(float (&a)[N], int lane) {
  static_assert(N >= (1 << NB), "tr_reduce: vector shorter than the lane group");
#pragma unroll
  for (int s = NB - 1; s >= 0; --s) {
    const int mask = 1 << (LB + s);
    const bool up = (lane & mask) != 0;
    const int half = (N >> (NB - 1 - s)) / 2;
    // bitwise blend: a conditional on the two elements is folded by the
    // compiler into a dynamically indexed read of the array (a select chain)
    const uint32_t m = up ? 0xffffffffu : 0u;
#pragma unroll
    for (int e = 0; e < half; ++e) {
      const uint32_t lo = __float_as_uint(a[e]), hi = __float_as_uint(a[e + half]);
      const float send = __uint_as_float((lo & m) | (hi & ~m));
      const float keep = __uint_as_float((hi & m) | (lo & ~m));
      a[e] = keep + __shfl_xor(send, mask);
    }
  }
}

// ------------------------------------------------------- buffer resources
// A raw buffer over [base, base + bytes): a load or store addresses it with
// one 32-bit lane offset (VGPR) plus a wave-uniform offset (SGPR), so a tile
// read row by row keeps a single address register per lane instead of one
// 64-bit pointer per row; accesses past the end are dropped by the hardware.
// Descriptor word 3 is the gfx9 raw-buffer format (0x00020000).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// Cache policy of the buffer accesses (aux operand): 0 the default, CP_NT
// non-temporal (the instruction's nt bit on gfx950).
constexpr int CP_NT = 2;
template <int N, int CP = 0>
__device__ __forceinline__ void buf_ld(__amdgpu_buffer_rsrc_t r, int voff, int soff, float (&x)[N]) {
  static_assert(N == 2 || N == 4, "buf_ld: 2 or 4 floats");
  if constexpr (N == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, CP);
    x[0] = __uint_as_float(v[0]); x[1] = __uint_as_float(v[1]);
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CP);
    x[0] = __uint_as_float(v[0]); x[1] = __uint_as_float(v[1]);
    x[2] = __uint_as_float(v[2]); x[3] = __uint_as_float(v[3]);
  }
}
template <int N, int CP = 0>
__device__ __forceinline__ void buf_st(__amdgpu_buffer_rsrc_t r, int voff, int soff, const float (&x)[N]) {
  static_assert(N == 2 || N == 4, "buf_st: 2 or 4 floats");
  if constexpr (N == 2) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    const u2 v = {__float_as_uint(x[0]), __float_as_uint(x[1])};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, soff, CP);
  } else {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, CP);
  }
}

// Two consecutive elements, rounded to T, stored through a buffer resource
// (fp32: 8 bytes; bf16: 4 bytes, packed).
template <typename T>
__device__ __forceinline__ void buf_st2(__amdgpu_buffer_rsrc_t r, int voff, int soff, const float (&x)[2]) {
  if constexpr (sizeof(T) == 4) {
    buf_st<2>(r, voff, soff, x);
  } else {
    const uint32_t v = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, 0);
  }
}

// ---------------------------------------------------------- DPP reductions
// Data-parallel-primitive moves read a neighbour lane's register inside the
// VALU instruction (no LDS permute, no address arithmetic).  Control codes
// (gfx9 encoding): quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_shl:n = 0x100 + n, row_mirror = 0x140, row_half_mirror = 0x141,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.  Lanes outside ROW_MASK, and
// lanes whose source lies outside the row, receive OLD.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float x, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xF, false));
}

// Sum over each row of 16 lanes; every lane of the row receives it.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x, 0.f);
  x += dpp_f<0x4E>(x, 0.f);
  x += dpp_f<0x141>(x, 0.f);
  x += dpp_f<0x140>(x, 0.f);
  return x;
}

// Product over each row of 16 lanes; every lane of the row receives it.
__device__ __forceinline__ float row16_prod(float x) {
  x *= dpp_f<0xB1>(x, 1.f);
  x *= dpp_f<0x4E>(x, 1.f);
  x *= dpp_f<0x141>(x, 1.f);
  x *= dpp_f<0x140>(x, 1.f);
  return x;
}

// Sum over each aligned group of N lanes (N = 1, 2, 4 or 8; lanes that
// differ in their low log2 N bits); every lane of the group receives it.
// The 8-lane step mirrors each half row, which pairs the two quads.
template <int N>
__device__ __forceinline__ float low_lane_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8, "low_lane_sum: 1, 2, 4 or 8 lanes");
  if constexpr (N >= 2) x += dpp_f<0xB1>(x, 0.f);
  if constexpr (N >= 4) x += dpp_f<0x4E>(x, 0.f);
  if constexpr (N >= 8) x += dpp_f<0x141>(x, 0.f);
  return x;
}

// Between a wave's LDS stores and its loads of values other lanes of the
// same wave stored: the wavefront-scope fences keep the compiler from moving
// the loads above the stores (the lanes' accesses do not alias from one
// lane's point of view), and the wave's LDS accesses then execute in order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Value of lane L (a compile-time or wave-uniform index) in every lane.
__device__ __forceinline__ float lane_value(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Sum over the 64 lanes of the wave, wave-uniform: row sums, then rows 0+1
// and 2+3 by row_bcast:15, all four by row_bcast:31, read from lane 63.
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += dpp_f<0x142, 0xA>(x, 0.f);
  x += dpp_f<0x143, 0xC>(x, 0.f);
  return lane_value(x, 63);
}

// Mamba-2 decay a = exp(-dt * exp(A)).
__device__ __forceinline__ float m2_decay(float dt, float A) { return __expf(-dt * __expf(A)); }

}  // namespace sk
