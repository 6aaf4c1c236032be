// Device helpers shared by the gfx950 kernels: storage types, bf16 <-> fp32,
// 16-byte vector loads, and DPP row reductions for 64-wide wavefronts.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "args.hpp"

namespace pkv {

// Storage tags: Elem<T>::kBytes, widening of 16 bytes into fp32 lanes.
struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16 bytes -> fp32 values (8 for bf16, 4 for fp32).
template <typename E> struct Vec;
template <> struct Vec<BF16> {
  static constexpr int kN = 8;
  __device__ __forceinline__ static void widen(const uint4 &x, float *f) {
    f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x);
    f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
    f[4] = bf16_lo(x.z); f[5] = bf16_hi(x.z);
    f[6] = bf16_lo(x.w); f[7] = bf16_hi(x.w);
  }
};
template <> struct Vec<F32> {
  static constexpr int kN = 4;
  __device__ __forceinline__ static void widen(const uint4 &x, float *f) {
    f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
    f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
  }
};

// A lane's 16-byte chunk of a query row, kept in the form the q.k dot
// product consumes: packed bf16 pairs (v_dot2_f32_bf16) or fp32.
template <typename E> struct QChunk;
template <> struct QChunk<BF16> {
  uint32_t w[4];
  __device__ __forceinline__ void set(const uint4 &x) { w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w; }
  // sum over the chunk of q * k, fp32 accumulation
  __device__ __forceinline__ float dot(const uint4 &k) const {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    float a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[0]),
                                              __builtin_bit_cast(bf16x2, k.x), 0.f, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[1]),
                                        __builtin_bit_cast(bf16x2, k.y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[2]),
                                        __builtin_bit_cast(bf16x2, k.z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[3]),
                                        __builtin_bit_cast(bf16x2, k.w), a, false);
    return a;
  }
};
template <> struct QChunk<F32> {
  float f[4];
  __device__ __forceinline__ void set(const uint4 &x) { Vec<F32>::widen(x, f); }
  __device__ __forceinline__ float dot(const uint4 &k) const {
    float a = f[0] * __uint_as_float(k.x);
    a = fmaf(f[1], __uint_as_float(k.y), a);
    a = fmaf(f[2], __uint_as_float(k.z), a);
    a = fmaf(f[3], __uint_as_float(k.w), a);
    return a;
  }
};

// Store n fp32 values as the storage type (bf16 by the hardware's
// round-to-nearest-even conversion). n a multiple of 8 (bf16) or 4 (fp32)
// with a 16-byte aligned destination uses 16-byte stores.
template <typename E> __device__ __forceinline__ void store_row(typename E::storage *dst, const float *v, int n);
template <> __device__ __forceinline__ void store_row<F32>(float *dst, const float *v, int n) {
  if ((n & 3) == 0) {
    for (int i = 0; i < n; i += 4)
      *reinterpret_cast<float4 *>(dst + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  } else {
    for (int i = 0; i < n; ++i) dst[i] = v[i];
  }
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
template <> __device__ __forceinline__ void store_row<BF16>(uint16_t *dst, const float *v, int n) {
  if ((n & 7) == 0) {
    for (int i = 0; i < n; i += 8) {
      uint4 w;
      w.x = pack_bf16x2(v[i], v[i + 1]);
      w.y = pack_bf16x2(v[i + 2], v[i + 3]);
      w.z = pack_bf16x2(v[i + 4], v[i + 5]);
      w.w = pack_bf16x2(v[i + 6], v[i + 7]);
      *reinterpret_cast<uint4 *>(dst + i) = w;
    }
  } else {
    for (int i = 0; i < n; ++i) dst[i] = (uint16_t)(pack_bf16x2(v[i], 0.f) & 0xffffu);
  }
}

template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N in {8, 16, 32}); every lane of the
// group gets the total. Fixed butterfly order, so results are repeatable.
template <int N> __device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of each 8
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror: other 8 of each 16
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load marked non-temporal (global_load_dwordx4 ... nt): the data is
// streamed once, and on gfx950 such loads sustain a markedly higher HBM
// read rate than ordinary cached loads.
__device__ __forceinline__ uint4 load_stream(const void *p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// A 16-byte K/V load: non-temporal (load_stream) for pages one request
// reads, or an ordinary cached load (C) for pages other requests of the call
// read too, so that they find them in L2. The policy is a compile-time
// choice: each loop streams with one kind of load.
template <bool C>
__device__ __forceinline__ uint4 load_kv(const void *p) {
  if constexpr (C) {
    return *reinterpret_cast<const uint4 *>(p);
  } else {
    return load_stream(p);
  }
}

}  // namespace pkv
