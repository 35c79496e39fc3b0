// Device-side building blocks shared by the gfx950 kernels: storage types,
// 16-byte row fragments, wavefront reductions and number conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

template <int DT> struct Elem;
template <> struct Elem<DT_F32>  { static constexpr int bytes = 4; };
template <> struct Elem<DT_F16>  { static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// 16-byte fragments: one lane's share of a K/V/q row
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Streaming load of K/V data: every byte is read once per decode step, so
// mark it non-temporal to keep it from displacing reusable lines.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 r;
  r.x = __builtin_nontemporal_load(&q->x);
  r.y = __builtin_nontemporal_load(&q->y);
  r.z = __builtin_nontemporal_load(&q->z);
  r.w = __builtin_nontemporal_load(&q->w);
  return r;
}

// Buffer descriptor over [base, base + bytes): loads through it take a
// wave-uniform base in scalar registers plus a 32-bit per-lane offset, and
// return 0 instead of touching memory outside the range.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                          0x00020000);
}
// 16-byte streaming (non-temporal) buffer load at base + soff + voff.
__device__ __forceinline__ uint4 ld16_buf(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
}

// 16-byte streaming buffer load written straight into LDS: lane l's bytes
// land at lds + 16*l (the address is wave-uniform and goes through M0).
__device__ __forceinline__ void ld16_buf_to_lds(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)voff, (int)soff, 0, 2);
}

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int vmcnt_only(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Dot product of a 16-byte K fragment with the matching q fragment, added
// to acc.  16-bit types use the packed two-way dot instructions (products of
// two 16-bit floats are exact in float32).
template <int DT>
__device__ __forceinline__ float dot16(const uint4& k, const uint4& q, float acc);

template <>
__device__ __forceinline__ float dot16<DT_BF16>(const uint4& k, const uint4& q, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                        __builtin_bit_cast(bf16x2_t, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                        __builtin_bit_cast(bf16x2_t, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                        __builtin_bit_cast(bf16x2_t, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                        __builtin_bit_cast(bf16x2_t, q.w), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float dot16<DT_F16>(const uint4& k, const uint4& q, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.x),
                               __builtin_bit_cast(f16x2_t, q.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.y),
                               __builtin_bit_cast(f16x2_t, q.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.z),
                               __builtin_bit_cast(f16x2_t, q.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, k.w),
                               __builtin_bit_cast(f16x2_t, q.w), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float dot16<DT_F32>(const uint4& k, const uint4& q, float acc) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

// two floats -> two packed 16-bit values (round to nearest even)
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == DT_F16)
    return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
  else
    return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}

// acc + a.lo * b.lo + a.hi * b.hi over two packed 16-bit values
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  acc, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// x rounded to the storage type (round to nearest even), as float32;
// float32 storage: x itself
template <int DT>
__device__ __forceinline__ float round_to(float x) {
  if constexpr (DT == DT_F16) return (float)(_Float16)x;
  else if constexpr (DT == DT_BF16) return (float)(__bf16)x;
  else return x;
}

// Widen a 16-byte fragment to float32 (exact for every storage type).
template <int DT>
__device__ __forceinline__ void widen16(const uint4& v, float* o);

template <>
__device__ __forceinline__ void widen16<DT_BF16>(const uint4& v, float* o) {
  o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
  o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
}
template <>
__device__ __forceinline__ void widen16<DT_F16>(const uint4& v, float* o) {
  o[0] = f16_lo(v.x); o[1] = f16_hi(v.x); o[2] = f16_lo(v.y); o[3] = f16_hi(v.y);
  o[4] = f16_lo(v.z); o[5] = f16_hi(v.z); o[6] = f16_lo(v.w); o[7] = f16_hi(v.w);
}
template <>
__device__ __forceinline__ void widen16<DT_F32>(const uint4& v, float* o) {
  o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
  o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}

// ---------------------------------------------------------------------------
// float32 -> storage type, round to nearest even
// ---------------------------------------------------------------------------
// float -> bf16 with round-to-nearest-even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

template <int DT>
__device__ __forceinline__ void store_elem(void* base, size_t idx, float x) {
  if constexpr (DT == DT_F32) {
    reinterpret_cast<float*>(base)[idx] = x;
  } else if constexpr (DT == DT_F16) {
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_f16_bits(x);
  } else {
    reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(x);
  }
}

// ---------------------------------------------------------------------------
// math
// ---------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh from its definition: tanh|x| = 1 - 2 / (e^{2|x|} + 1), sign restored.
// Absolute error is a few float32 ulps of 1.
__device__ __forceinline__ float tanh_def(float x) {
  float ax = fabsf(x);
  float e = fast_exp2(ax * (2.0f * kLog2e));
  float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  return copysignf(t, x);
}

// ---------------------------------------------------------------------------
// wavefront reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// v from lane (lane ^ mask).  Masks 1, 2 and 8 stay inside a 16-lane row
// and use DPP (quad permute, row rotate by 8); 4 and 16 use the LDS-free
// swizzle network; 32 uses the lane permute crossbar.  `mask` is a
// compile-time constant after unrolling, so the chain folds to one case.
__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  const int x = __float_as_int(v);
  int r;
  if (mask == 1) r = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);        // quad_perm 1,0,3,2
  else if (mask == 2) r = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  else if (mask == 8) r = __builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror 8
  else if (mask == 4) r = __builtin_amdgcn_ds_swizzle(x, 0x1F | (4 << 10));
  else if (mask == 16) r = __builtin_amdgcn_ds_swizzle(x, 0x1F | (16 << 10));
  else r = __builtin_amdgcn_ds_bpermute((lane_id() ^ mask) << 2, x);
  return __int_as_float(r);
}

// Reduce-scatter of N independent partial sums across the LPR lanes of an
// aligned lane group.  Step by step (masks LPR/2 .. 1) each lane keeps half
// of its values and adds the partner's copy of that half, so every shuffle
// moves useful data.  Afterwards lane holds max(1, N/LPR) complete sums in
// v[0..): those with indices tr_base(lane) + t.  When N < LPR the last steps
// are plain butterflies and neighbouring lanes hold the same sum.
template <int CUR, int M, int N>
struct TransposeReduce {
  static __device__ __forceinline__ void run(float (&v)[N], int lane) {
    if constexpr (M >= 1) {
      if constexpr (CUR > 1) {
        constexpr int H = CUR / 2;
        const bool up = (lane & M) != 0;
#pragma unroll
        for (int j = 0; j < H; ++j) {
          float send = up ? v[j] : v[j + H];
          float keep = up ? v[j + H] : v[j];
          v[j] = keep + shfl_xor_f(send, M);
        }
        TransposeReduce<H, M / 2, N>::run(v, lane);
      } else {
        v[0] += shfl_xor_f(v[0], M);
        TransposeReduce<1, M / 2, N>::run(v, lane);
      }
    }
  }
};

template <int N, int LPR>
__device__ __forceinline__ int tr_base(int lane) {
  int base = 0;
  int cur = N;
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) {
    if (cur > 1) {
      cur >>= 1;
      if (lane & m) base += cur;
    }
  }
  return base;
}

}  // namespace pa
