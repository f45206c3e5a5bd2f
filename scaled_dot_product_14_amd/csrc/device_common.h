// Device helpers for the gfx950 (CDNA4) attention kernels: bf16 / fp16 MFMA tiles,
// LDS transposed reads and cross-half wavefront exchange.
//
// Lane layouts used throughout (wave64, checked on gfx950):
//   v_mfma_f32_32x32x16_bf16  C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row l%32, k = 8*(l/32) + 0..7 (8 bf16)
//     B: lane l holds col l%32, k = 8*(l/32) + 0..7 (8 bf16)
//     C: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, col l%32
//   ds_read_b64_tr_b16 (16-lane groups): lane j of a group receives element
//     j%4 of the 4 x 16-bit words addressed by lanes 4*i + j/4, i = 0..3.  When
//     lane j addresses row r0 + j/4, columns c0 + 4*(j%4) .. +3 of a row-major
//     16-bit matrix, lane j receives column c0 + j, rows r0 .. r0+3: a
//     transposed 4x16 read.
//   permlane32_swap(x, x) gives {x[l], x[l+32]} on lanes < 32 and
//     {x[l-32], x[l]} on lanes >= 32, so combining both halves of the result
//     reduces over the lane pair (l, l^32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa14 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Reads one dword of every 64-byte line of the first BYTES bytes of the
// kernel's arguments (at most eight lines), as one batch of scalar loads with
// a single wait.  The argument loads the code issues afterwards then hit the
// scalar cache; left alone they come in rounds (the tile's coordinates first,
// then the pointers and strides the tile needs), each a memory round trip at
// a kernel's start.
// `also` joins the batch: an argument the caller reads at an index of its
// own (a table entry picked by the workgroup index) costs no extra round trip.
template <int BYTES>
__device__ __forceinline__ void warm_kernargs(uint32_t also = 0u) {
  static_assert(BYTES > 0 && BYTES <= 8 * 64, "one to eight lines");
  const uint32_t __attribute__((address_space(4)))* ka =
      (const uint32_t __attribute__((address_space(4)))*)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = i * 64 < BYTES ? ka[i * 16] : 0u;
  asm volatile("" ::"s"(x[0]), "s"(x[1]), "s"(x[2]), "s"(x[3]), "s"(x[4]), "s"(x[5]), "s"(x[6]),
               "s"(x[7]), "s"(also));
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.f;
  return z;
}

// 16-byte global load of 8 bf16.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// 16-byte LDS load of 8 bf16.
__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposed 64-bit LDS read (see the layout note above).
__device__ __forceinline__ bf16x4 lds_tr4(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 concat(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Maximum / sum over the lane pair (l, l^32).
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Bitwise or over the lane pair (l, l^32).
__device__ __forceinline__ uint32_t pair_or(uint32_t x) {
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] | r[1];
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over `bytes` bytes at `base`: 16-byte loads at offsets at
// or past the end return zeros instead of touching memory (the range check of
// the buffer unit), which replaces per-lane bounds branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// acc + sum_i x[i] * y[i] over 8 bf16 pairs (v_dot2_f32_bf16, fp32 accumulate).
__device__ __forceinline__ float dot8_bf16(const bf16x8& x, const bf16x8& y, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1),
                                        __builtin_shufflevector(y, y, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3),
                                        __builtin_shufflevector(y, y, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5),
                                        __builtin_shufflevector(y, y, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7),
                                        __builtin_shufflevector(y, y, 6, 7), acc, false);
  return acc;
}

// Round four floats to bf16 (nearest even) and pack them into 8 bytes.
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  v[2] = (__bf16)c;
  v[3] = (__bf16)d;
  return __builtin_bit_cast(uint2, v);
}

// ---- 16-bit element formats ----------------------------------------------
// Fragments travel as bf16x8 / bf16x4 bit containers whatever the format; the
// F16 flag picks IEEE half instead of bfloat16 where values are multiplied or
// converted.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <bool F16>
__device__ __forceinline__ f32x16 mfma16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// float -> 16-bit value (round to nearest even), as a bit container.
template <bool F16>
__device__ __forceinline__ __bf16 to16(float x) {
  if constexpr (F16)
    return __builtin_bit_cast(__bf16, static_cast<_Float16>(x));
  else
    return static_cast<__bf16>(x);
}

// The 16-bit value in the low half of `bits` -> float.
template <bool F16>
__device__ __forceinline__ float from16(uint32_t bits) {
  if constexpr (F16)
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
  else
    return __uint_as_float(bits << 16);
}

template <bool F16>
__device__ __forceinline__ uint2 pack16x4(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = to16<F16>(a);
  v[1] = to16<F16>(b);
  v[2] = to16<F16>(c);
  v[3] = to16<F16>(d);
  return __builtin_bit_cast(uint2, v);
}

// acc + sum_i x_i * y_i over 8 16-bit values, fp32 accumulation.
template <bool F16>
__device__ __forceinline__ float dot8_16(const bf16x8& x, const bf16x8& y, float acc) {
  if constexpr (F16) {
    const f16x8 a = __builtin_bit_cast(f16x8, x), b = __builtin_bit_cast(f16x8, y);
#pragma unroll
    for (int i = 0; i < 8; i += 2)
      acc = __builtin_amdgcn_fdot2(f16x2{a[i], a[i + 1]}, f16x2{b[i], b[i + 1]}, acc, false);
    return acc;
  } else {
    return dot8_bf16(x, y, acc);
  }
}

// Within-row lane permutations (DPP): xor 1, xor 2 (quad_perm), and the
// mirrors of each 8-lane half row and of the 16-lane row.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of N lanes (N = 8 or 16), result in every lane of the group.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp_move<kDppXor1>(x);
  x += dpp_move<kDppXor2>(x);
  x += dpp_move<kDppHalfMirror>(x);
  if (N == 16) x += dpp_move<kDppMirror>(x);
  return x;
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// Waits here for the load that produced x.  A register loaded before a loop
// and first read inside it otherwise stays "in flight" at the loop header in
// the compiler's wait bookkeeping, and every iteration then waits for all
// loads issued before that read, prefetches included.
__device__ __forceinline__ void settle(const bf16x8& x) { asm volatile("" ::"v"(x)); }

}  // namespace sdpa14
