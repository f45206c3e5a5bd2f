// LDS staging helpers shared by the attention kernels: XOR-swizzled tiles,
// buffer loads that write LDS directly, and the barrier of a staging ring.
#pragma once

#include "device_common.h"

namespace sdpa14 {

// A staged tile holds 32 rows of E bf16, 2E bytes per row, no padding.  The
// 16-byte chunk c of row r sits at chunk position c ^ tile_swz(r).  The
// permutation keeps the two read patterns free of LDS bank conflicts: the
// row-per-lane 16-byte reads (16 consecutive rows, one chunk) and the
// transposed 8-byte reads (4 consecutive rows x 4 aligned chunks).
template <int E>
__device__ __forceinline__ int tile_swz(int r) {
  return E == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3)) : (((r & 3) << 2) | ((r >> 2) & 3));
}

// s_waitcnt with vmcnt <= VM and lgkmcnt == 0 (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt in 6:4 left at its maximum, lgkmcnt in 11:8).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

// Workgroup barrier of the LDS ring.  Each wave first waits until at most VM
// of its loads are in flight (the older ones, which fill the next stage, have
// landed in LDS) and its LDS reads have returned.  The empty asm statements
// keep the compiler from moving LDS accesses across the barrier.
template <int VM>
__device__ __forceinline__ void ring_barrier() {
  asm volatile("" ::: "memory");
  wait_vm_lgkm0<VM>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte buffer load per lane into LDS: lane l writes lds_wave + 16*l.
// lds_wave must be wave-uniform.  Out-of-range offsets deliver zeros.  Issued
// from inline assembly so that the compiler's wait bookkeeping does not tie
// later LDS reads of other stages to these loads; the ring barrier waits for
// them explicitly.  M0 carries the LDS address (the compiler sets M0 afresh
// before each of its own uses); an LDS-DMA instruction needs one wait state
// after the SALU write of M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is a reserved register
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds_wave,
                                      uint32_t voff) {
  const uint32_t dst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(dst), "v"(voff), "s"(r)
               : "m0");
}
// The same load, ordered after the computation of `after` (an unused operand),
// so the compiler cannot hoist it above that point.
__device__ __forceinline__ void dma16_after(__amdgpu_buffer_rsrc_t r, unsigned char* lds_wave,
                                            uint32_t voff, float after) {
  const uint32_t dst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(dst), "v"(voff), "s"(r), "v"(after)
               : "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int rows,
                                                            int64_t stride, int E) {
  return make_rsrc(base, rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * stride + E) * 2) : 0u);
}

// Per-thread part of a tile load by NT threads: load k of thread tid fills
// slot k*NT + tid, i.e. row slot/CPR at chunk position slot%CPR, which holds
// the global chunk (slot%CPR) ^ tile_swz(row).  Returns the byte offset from
// the tile's first row.
template <int E, int NT = 256>
__device__ __forceinline__ uint32_t dma_src_offset(int k, int tid, int64_t row_stride) {
  constexpr int CPR = E / 8;
  const int slot = k * NT + tid;
  const int row = slot / CPR, pos = slot % CPR;
  return (uint32_t)row * (uint32_t)(row_stride * 2) + (uint32_t)((pos ^ tile_swz<E>(row)) * 16);
}

// The same offset for a tile whose rows hold only the first e_real of their E
// elements (e_real a multiple of 8): a chunk past e_real gets bit 31 set.  A
// (batch, head) slice stays below 2 GiB, so the buffer range check turns that
// load into zeros, and adding a row offset below 2^31 keeps the bit.
template <int E, int NT = 256>
__device__ __forceinline__ uint32_t dma_src_offset_e(int k, int tid, int64_t row_stride,
                                                     int e_real) {
  constexpr int CPR = E / 8;
  const int slot = k * NT + tid;
  const int row = slot / CPR, pos = slot % CPR;
  const int chunk = pos ^ tile_swz<E>(row);
  return ((uint32_t)row * (uint32_t)(row_stride * 2) + (uint32_t)(chunk * 16)) |
         (chunk * 8 < e_real ? 0u : 0x80000000u);
}

// LDS byte offset, within a tile, of the chunk holding elements 8c .. 8c+7 of row r.
template <int E>
__device__ __forceinline__ int chunk_off(int r, int c) {
  return r * (2 * E) + ((c ^ tile_swz<E>(r)) << 4);
}

// LDS byte offset, within a tile, of elements e .. e+3 of row r (e % 4 == 0),
// the 8 bytes one lane addresses in a transposed read.
template <int E>
__device__ __forceinline__ int tr_off(int r, int e) {
  return r * (2 * E) + (((e >> 3) ^ tile_swz<E>(r)) << 4) + ((e & 4) << 1);
}

// Byte offset of ring stage it % NSTAGE as one wave-uniform scalar, so that LDS
// addresses are a per-lane base plus this offset plus an immediate.
template <int STAGE, int NSTAGE = 3>
__device__ __forceinline__ uint32_t ring_offset(int it) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((it % NSTAGE) * STAGE);
}

template <typename T>
__device__ __forceinline__ T lds_at(const unsigned char* base, int off) {
  return *reinterpret_cast<const T*>(base + off);
}

__device__ __forceinline__ bf16x8 tr_pair(const unsigned char* tile, int o0, int o1) {
  return concat(lds_tr4(reinterpret_cast<const uint16_t*>(tile + o0)),
                lds_tr4(reinterpret_cast<const uint16_t*>(tile + o1)));
}

}  // namespace sdpa14
