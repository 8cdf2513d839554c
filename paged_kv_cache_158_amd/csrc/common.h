// Device helpers shared by the gfx950 kernels: bf16 packing, cross-lane
// moves inside a 64-lane wavefront, and small integer utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ uint32_t word(const u32x4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two fp32 values rounded to bf16 (nearest-even, v_cvt_pk_bf16_f32), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs, fp32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// (lo half of a, lo half of b) and (hi half of a, hi half of b) as bf16 pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// --- cross-lane moves -------------------------------------------------------
// DPP controls (GCN3+/CDNA encoding).
enum : int {
  DPP_QUAD_XOR1 = 0xB1,       // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,       // quad_perm [2,3,0,1]
  DPP_ROW_ROR8 = 0x128,       // row_ror:8 == lane ^ 8 inside a 16-lane row
  DPP_ROW_HALF_MIRROR = 0x141 // lane ^ 7 inside each 8-lane half row
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), CTRL, 0xF, 0xF, false));
}

// x from lane (lane ^ X) for X in {1, 2, 7, 8, 16, 32}; each pairing stays
// inside the aligned group of size 2, 4, 8, 16, 32, 64 respectively.
template <int X>
__device__ __forceinline__ float xor_lane(float x) {
  if constexpr (X == 1) return dpp_f32<DPP_QUAD_XOR1>(x);
  else if constexpr (X == 2) return dpp_f32<DPP_QUAD_XOR2>(x);
  else if constexpr (X == 7) return dpp_f32<DPP_ROW_HALF_MIRROR>(x);
  else if constexpr (X == 8) return dpp_f32<DPP_ROW_ROR8>(x);
  else if constexpr (X == 16)
    // ds_swizzle bit mode: and_mask 0x1f, or_mask 0, xor_mask 0x10
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (0x10 << 10) | 0x1F));
  else {
    static_assert(X == 32, "unsupported lane xor");
    return __shfl_xor(x, 32, 64);
  }
}

// Value of lane (group_base + SRC) where group_base = lane & ~(W-1), for a
// group width W in {8, 16, 32}.
template <int W, int SRC>
__device__ __forceinline__ uint32_t bcast_in_group(uint32_t x) {
  static_assert(SRC >= 0 && SRC < W, "source lane outside group");
  if constexpr (W == 16)
    return dpp_u32<0x150 + SRC>(x);  // row_newbcast:SRC
  else {
    static_assert(W == 8 || W == 32, "unsupported group width");
    constexpr int and_mask = 0x1F & ~(W - 1);
    return static_cast<uint32_t>(
        __builtin_amdgcn_ds_swizzle(static_cast<int>(x), (SRC << 5) | and_mask));
  }
}

template <int W, int SRC>
__device__ __forceinline__ float bcast_in_group_f(float x) {
  return __uint_as_float(bcast_in_group<W, SRC>(__float_as_uint(x)));
}

__host__ __device__ constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// 0 in a vector register, opaque to the compiler: adding it to an index
// makes a load of one uniform address a vector load (counted with the other
// vector loads) instead of a scalar one, whose counter the LDS reads of the
// same wave would have to wait on.
__device__ __forceinline__ int vgpr_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

constexpr float kLog2e = 1.4426950408889634f;

// Rotated cache layout: inside a slot, KV head h of the token at in-block
// position p is stored at head position (h + p) mod H_kv when H_kv is a
// power of two (at h otherwise).  A wave reading one head over consecutive
// tokens then touches every head position of the slot rows instead of
// always the same byte offset, which spreads its reads evenly over the HBM
// address interleave.  rot = H_kv - 1 for a power of two, else 0; the plain
// layout is rot = 0 (kv_head_pos(h, p, 0) = h).
__host__ __device__ constexpr int kv_rot_mask(int num_kv_heads) {
  return (num_kv_heads & (num_kv_heads - 1)) == 0 ? num_kv_heads - 1 : 0;
}
__host__ __device__ __forceinline__ int kv_head_pos(int h, int p, int rot) {
  return ((h + p) & rot) | (h & ~rot);
}

// 8 bf16 values (element order kept) -> 8 E4M3 codes: the nearest code to
// x / s in float32, ties to even, after clamping to +-448 (the conversion
// instruction turns larger magnitudes into NaN); a NaN x gives the NaN code
// 0x7F with the sign bit of x.  Shared by every FP8 cache write so that
// they give the same codes.
__device__ __forceinline__ uint2 quant_fp8x8(const u32x4& x, float s) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float f[4];
    uint32_t nan_code = 0, keep = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t word = w[2 * q + (i >> 1)];
      const uint32_t b = (i & 1) ? (word >> 16) : (word & 0xFFFFu);  // bf16 bits
      f[i] = fminf(fmaxf(__uint_as_float(b << 16) / s, -448.f), 448.f);
      const bool nan = (b & 0x7FFFu) > 0x7F80u;
      nan_code |= nan ? (0x7Fu | ((b >> 8) & 0x80u)) << (8 * i) : 0u;
      keep &= nan ? ~(0xFFu << (8 * i)) : 0xFFFFFFFFu;
    }
    uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], r, true);
    o[q] = (r & keep) | nan_code;
  }
  return make_uint2(o[0], o[1]);
}

}  // namespace pa
