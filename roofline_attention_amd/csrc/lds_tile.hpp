// LDS tile staging shared by the gfx950 attention kernels: direct buffer loads from HBM into
// LDS, XOR-swizzled tile layouts, and the transposing LDS read.
//
// A wave's buffer_load_dwordx4 ... lds instruction writes 64 x 16 bytes to one contiguous 1 KB
// block of LDS in lane order, so tiles cannot be padded; bank conflicts are avoided instead by
// storing the 16-byte chunk c of tile row r at chunk position c ^ swz(r). The swizzles:
//   swz_rows(r) = r mod CH           row-operand reads: 32 lanes read one chunk of 32 rows;
//   swz_tr(r)                        transposed reads: 32 lanes read 4 rows x 4 chunks;
//   swz_both(r)                      a tile read both ways.
// (CH = 16-byte chunks per row.) ds_read_b64_tr_b16 serves 32 lanes per LDS cycle across 64
// banks, so the 4 rows of a transposed read must fall in distinct 4-chunk blocks.
#pragma once

#include "common.hpp"

namespace ra {

typedef void __attribute__((address_space(3))) * lds_void_ptr;
typedef bf16x4 __attribute__((address_space(3))) * lds_bf16x4_ptr;

template <int HD>
__device__ __forceinline__ int swz_rows(int r) { return r & (HD / 8 - 1); }

template <int HD>
__device__ __forceinline__ int swz_tr(int r) {
  if constexpr (HD == 128) return 4 * (r & 3) + 2 * ((r >> 1) & 1);
  else return (2 * r) & 7;
}

template <int HD>
__device__ __forceinline__ int swz_both(int r) {
  return (4 * (r & 3) + ((r >> 2) & 3)) & (HD / 8 - 1);
}

// s_waitcnt immediate that waits until at most `vm` vector-memory operations of this wave are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at their maxima).
constexpr int waitcnt_vm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Raw buffer resource over `bytes` bytes from `base`; loads at or beyond `bytes` return zero
// without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes < 0 ? 0 : bytes, 0x00020000);
}

// Direct load into LDS: lane i of the wave writes lds_block + SIZE * i with the SIZE bytes at
// byte offset voffset of the resource.
template <int SIZE>
__device__ __forceinline__ void load_to_lds(__amdgpu_buffer_rsrc_t rsrc, int voffset, void* lds_block) {
  static_assert(SIZE == 16 || SIZE == 4, "dwordx4 or dword");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)lds_block, 16, voffset, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)lds_block, 4, voffset, 0, 0, 0);
}

// Transposing read: in each 16-lane group, lane 4e + j supplies the address of 4 bf16 at row e
// of a 4-row block; lane i of the group receives the 4 elements of column i of that block.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p));
}

// The same read issued as inline assembly. The compiler's wait insertion treats the builtin form
// as aliasing every direct-to-LDS load still in flight and waits for all of them (vmcnt(0)); a
// kernel that keeps the next tile's loads in flight across its reads of the current tile uses this
// form instead and orders it itself: the result may be used only after lds_wait(), which waits
// for all of this wave's LDS reads and ties the results so that no use is scheduled earlier.
__device__ __forceinline__ bf16x4 lds_read_tr_async(const bf16* p) {
  bf16x4 r;
  const unsigned addr = (unsigned)(uintptr_t)((const bf16 __attribute__((address_space(3)))*)p);
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

__device__ __forceinline__ bf16x8 tr_pair_async(const bf16* p0, const bf16* p1) {
  return __builtin_shufflevector(lds_read_tr_async(p0), lds_read_tr_async(p1), 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int N>
__device__ __forceinline__ void lds_wait_all(bf16x8 (&a)[N]) {
  static_assert(N == 4 || N == 8, "operand batch");
  if constexpr (N == 4) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]),
                 "+v"(a[6]), "+v"(a[7]));
  }
}

// Stages ROWS x HD bf16 rows [row0, row0 + ROWS) of a row-major [n_rows, HD] matrix into an LDS
// tile with swizzle SWZ; rows at or beyond n_rows read as zero. Called by all NWAVES waves of
// the workgroup, wave w issuing the 1 KB blocks w, w + NWAVES, ...
template <int HD, int ROWS, int NWAVES, int (*SWZ)(int)>
__device__ __forceinline__ void stage_tile(const bf16* __restrict__ src, int row0, int n_rows, bf16* tile, int w,
                                           int lane) {
  constexpr int CH = HD / 8;
  constexpr int RPI = 1024 / (HD * 2);
  constexpr int BLOCKS = ROWS / RPI;
  static_assert(BLOCKS % NWAVES == 0, "tile geometry");
  const auto rsrc = make_rsrc(src + (size_t)row0 * HD, (n_rows - row0) * HD * 2);
#pragma unroll
  for (int u = 0; u < BLOCKS / NWAVES; ++u) {
    const int blk = u * NWAVES + w;
    const int row = blk * RPI + lane / CH;
    load_to_lds<16>(rsrc, (row * HD + (((lane % CH) ^ SWZ(row)) * 8)) * 2, tile + blk * RPI * HD);
  }
}

// Address of the 16-byte chunk `chunk` of row `row` in a tile with swizzle SWZ.
template <int HD, int (*SWZ)(int)>
__device__ __forceinline__ const bf16* tile_chunk(const bf16* tile, int row, int chunk) {
  return tile + row * HD + ((chunk ^ SWZ(row)) * 8);
}

}  // namespace ra
