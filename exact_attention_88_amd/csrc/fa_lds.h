// LDS tile layout and global -> LDS loads shared by the tuned 16-bit kernels
// (fa_fwd_f16.hip, fa_bwd_f16.hip, fa_bwd_split.hip).
//
// Tiles are rows of D 16-bit elements (D = 128: 256 bytes, D = 64: 128
// bytes) stored unpadded in an XOR-swizzled layout that one copy serves for
// both row-wise MFMA operand reads (ds_read_b128) and transposed ones
// (ds_read_b64_tr_b16), and are filled either through registers or straight
// from global memory with buffer loads that write LDS.
#pragma once

#include "fa_common.h"

namespace fa {
namespace swzl {

constexpr int kD = 128;  // default elements per tile row

// Single-copy swizzled layout: unpadded rows in which the 16-byte chunk k of
// row r sits at chunk position k ^ swz<D>(r).  LDS serves 64 four-byte banks,
// i.e. 16 chunk positions per 256 bytes.
//   D = 128 (16 chunks a row): swz(r) takes distinct values on any 16
//   consecutive rows (16-row ds_read_b128 reads of one chunk and full-row
//   stores are conflict free) and, on 4 rows that start at a multiple of 4,
//   spreads 4 neighbouring chunks over all 16 chunk positions (4-row
//   transposed reads are conflict free).
//   D = 64 (8 chunks, two rows per 256 bytes): the row's parity picks the
//   bank half, and swz(r) in 0..7 is distinct over the 8 even and over the 8
//   odd rows of any 16 aligned rows (row reads) and differs in bit 2 between
//   rows 4i and 4i+2 (and 4i+1, 4i+3), so 4 aligned rows x 4 neighbouring
//   chunks (a transposed read) cover all 16 positions.
// Either way swz has period 16 in r.
template <int D = kD>
__device__ __forceinline__ int swz(int r) {
  static_assert(D == 128 || D == 64, "tuned tiles are 64 or 128 elements wide");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

template <int ROWS, int NT, class T>
__device__ __forceinline__ void tile_store_swz(const u32x4* r, T* lds) {
  constexpr int PER = ROWS * 16 / NT;
  static_assert(NT % 256 == 0, "every thread keeps its row residue mod 16");
  const int row0 = (int)threadIdx.x >> 4, off = row0 * kD + (((threadIdx.x & 15) ^ swz(row0)) << 3);
#pragma unroll
  for (int i = 0; i < PER; ++i) *reinterpret_cast<u32x4*>(lds + i * (NT / 16) * kD + off) = r[i];
}

// Row-wise fragment in the swizzled layout; rbase is a multiple of 16.
template <class T, int D = kD>
__device__ __forceinline__ V8<T> frag_r_swz(const T* lds, int rbase, int kchunk) {
  const int lane = threadIdx.x & 63, r = lane & 31;
  return *reinterpret_cast<const V8<T>*>(lds + (rbase + r) * D +
                                      (((kchunk + (lane >> 5)) ^ swz<D>(r)) << 3));
}

// Transposed fragment in the swizzled layout (same lanes as frag_t); rbase is
// a multiple of 16 and cbase of 8.
template <class T, int D = kD>
__device__ __forceinline__ V8<T> frag_t_swz(const T* lds, int rbase, int t, int cbase) {
  const int lane = threadIdx.x & 63, g = lane >> 5, j = lane & 15;
  const int col = ((lane >> 4) & 1) * 16 + (j & 3) * 4;
  const int r = g * 4 + (j >> 2);
  const int ch = (cbase >> 3) + (col >> 3);
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const T* p0 = lds + (rbase + t * 16 + r) * D + ((ch ^ swz<D>(r)) << 3) + (col & 7);
  const T* p1 = lds + (rbase + t * 16 + r + 8) * D + ((ch ^ swz<D>(r + 8)) << 3) + (col & 7);
  s4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
  s4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p1));
  V4<T> ah = __builtin_bit_cast(V4<T>, a), bh = __builtin_bit_cast(V4<T>, b);
  V8<T> x;
  x[0] = ah[0]; x[1] = ah[1]; x[2] = ah[2]; x[3] = ah[3];
  x[4] = bh[0]; x[5] = bh[1]; x[6] = bh[2]; x[7] = bh[3];
  return x;
}


template <bool V> struct BoolTag { static constexpr bool value = V; };
typedef int rsrc_t __attribute__((ext_vector_type(4)));  // buffer resource (4 SGPRs)

// Raw buffer over [base, base + nbytes): stride 0, 32-bit data format.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int nbytes) {
  const uint64_t p = (uint64_t)base;
  rsrc_t r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(p & 0xffffffffu));
  r[1] = __builtin_amdgcn_readfirstlane((int)((p >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(nbytes);
  r[3] = 0x00020000;
  return r;
}

// LDS byte address of a pointer into a __shared__ array (the m0 operand of
// buffer loads into LDS).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// One wave-wide 16-byte-per-lane buffer load into LDS at byte address m0
// (wave-uniform): lane i's bytes land at m0 + 16*i.  Issued as inline
// assembly so that the compiler does not make every later LDS read wait for
// it: the caller waits (vmcnt(0)) before the barrier that publishes the data.
__device__ __forceinline__ void dma16(rsrc_t r, unsigned m0, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voff), "s"(r) : "memory", "m0");
}

// tile_dma moves ROWS rows of D 16-bit elements into the swizzled layout with
// wave-wide 1 KB loads shared by the NW waves, each covering RL = 1024 / (2D)
// rows (D = 128: 4 rows of 16 chunks, D = 64: 8 rows of 8 chunks): load i of
// wave w covers tile rows (i*NW + w)*RL .. +RL-1; lane l takes row
// (i*NW + w)*RL + l/C (C = D/8 chunks a row), fetches that row's 16-byte chunk
// (l%C) ^ swz(row) and writes it at chunk position l%C (so chunk k sits at
// position k ^ swz(row)).  When NW*RL is a multiple of 16 every load moves the
// rows by a multiple of swz's period, so a lane's global byte offset is a
// per-lane part fixed for the kernel (dma_lane_off, for row stride ss_bytes)
// plus a wave-uniform row offset: one vector add per load.
template <int D>
constexpr int dma_rows() { return 1024 / (2 * D); }

template <int NW, int D = kD>
__device__ __forceinline__ int dma_lane_off(int ss_bytes) {
  constexpr int RL = dma_rows<D>(), C = D / 8;
  static_assert((NW * RL) % 16 == 0, "loads move whole multiples of 16 rows");
  const int lane = threadIdx.x & 63, row = ((int)threadIdx.x >> 6) * RL + lane / C;
  return row * ss_bytes + (((lane % C) ^ swz<D>(row)) << 4);
}

// ROWS rows starting at global row row0 into the tile at LDS byte address lds
// (wave-uniform).  The caller guarantees that every byte offset fits in 31
// bits; rows past the buffer's byte range read as zero.
template <int ROWS, int NW, int D = kD>
__device__ __forceinline__ void tile_dma(rsrc_t r, unsigned lds, int lane_off, int ss_bytes, int row0) {
  constexpr int RL = dma_rows<D>();
  static_assert(ROWS % (RL * NW) == 0 && (NW * RL) % 16 == 0, "whole wave loads of 16-row multiples");
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < ROWS / (RL * NW); ++i)
    dma16(r, lds + (unsigned)((i * NW + w) * 1024), lane_off + (row0 + i * NW * RL) * ss_bytes);
}

}  // namespace swzl
}  // namespace fa
