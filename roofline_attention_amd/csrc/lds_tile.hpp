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

// The same resource as its four descriptor words (base address, stride 0, byte count, raw-buffer
// flags), wave-uniform, for the direct-to-LDS loads below.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)(bytes < 0 ? 0 : bytes));
  r[3] = 0x00020000u;
  return r;
}

// Direct load into LDS: lane i of the wave writes lds_block + SIZE * i with the SIZE bytes at byte
// offset voffset of the resource (buffer_load_dword[x4] ... lds; M0 holds the LDS block address,
// which must be wave-uniform). Issued as inline assembly on purpose: the compiler's wait insertion
// models the builtin form as a write that may alias every later LDS read and waits for all such
// loads in flight (vmcnt(0)) before the next LDS read, which would expose the latency of a tile
// prefetched across the reads of the current one. Callers therefore order these loads
// themselves: a tile is read only after s_waitcnt vmcnt(0) and a workgroup barrier.
template <int SIZE>
__device__ __forceinline__ void load_to_lds(const u32x4& rsrc, int voffset, const void* lds_block) {
  static_assert(SIZE == 16 || SIZE == 4, "dwordx4 or dword");
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_block;
  if constexpr (SIZE == 16)
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(rsrc), "{m0}"(m0) : "memory");
  else
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voffset), "s"(rsrc), "{m0}"(m0) : "memory");
}

// The same 16-byte load with a wave-uniform byte offset `soffset` added in the instruction's scalar
// offset operand: a wave's blocks that sit a fixed (uniform) distance apart share one per-lane
// voffset register instead of one each.
__device__ __forceinline__ void load_to_lds16_so(const u32x4& rsrc, int voffset, int soffset, const void* lds_block) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_block;
  asm volatile("buffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voffset), "s"(rsrc), "{m0}"(m0),
               "s"(__builtin_amdgcn_readfirstlane(soffset))
               : "memory");
}

// Transposing read: in each 16-lane group, lane 4e + j supplies the address of 4 bf16 at row e
// of a 4-row block; lane i of the group receives the 4 elements of column i of that block.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p));
}

// Bytes of the rows [row0, row0 + ROWS) of a [n_rows, HD] bf16 matrix that exist: the byte count
// of a staged tile's buffer resource. Only the tile's own rows count, so the value is at most
// ROWS * HD * 2 and never overflows int (n_rows * HD * 2 itself reaches 2^31 at n_rows * HD = 2^30,
// the largest size the library accepts).
template <int HD, int ROWS>
__host__ __device__ constexpr int tile_span_bytes(int n_rows, int row0) {
  return (n_rows - row0 <= 0 ? 0 : (n_rows - row0 < ROWS ? n_rows - row0 : ROWS)) * HD * 2;
}
static_assert(tile_span_bytes<128, 64>(1 << 23, 0) == 64 * 128 * 2, "first tile at N * d = 2^30");
static_assert(tile_span_bytes<64, 64>(1 << 24, 0) == 64 * 64 * 2, "first tile at N * d = 2^30");
static_assert(tile_span_bytes<128, 64>((1 << 23), (1 << 23) - 10) == 10 * 128 * 2, "ragged last tile");
static_assert(tile_span_bytes<128, 64>(100, 128) == 0, "tile past the end");

// Stages ROWS x HD bf16 rows [row0, row0 + ROWS) of a row-major [n_rows, HD] matrix into an LDS
// tile with swizzle SWZ; rows at or beyond n_rows read as zero. Called by all NWAVES waves of
// the workgroup, wave w issuing the 1 KB blocks w, w + NWAVES, ... The buffer resource covers
// only the tile's own rows (tile_span_bytes).
template <int HD, int ROWS, int NWAVES, int (*SWZ)(int)>
__device__ __forceinline__ void stage_tile(const bf16* __restrict__ src, int row0, int n_rows, bf16* tile, int w,
                                           int lane) {
  constexpr int CH = HD / 8;
  constexpr int RPI = 1024 / (HD * 2);
  constexpr int BLOCKS = ROWS / RPI;
  static_assert(BLOCKS % NWAVES == 0, "tile geometry");
  const u32x4 rsrc = dma_rsrc(src + (size_t)row0 * HD, tile_span_bytes<HD, ROWS>(n_rows, row0));
#pragma unroll
  for (int u = 0; u < BLOCKS / NWAVES; ++u) {
    const int blk = u * NWAVES + w;
    const int row = blk * RPI + lane / CH;
    load_to_lds<16>(rsrc, (row * HD + (((lane % CH) ^ SWZ(row)) * 8)) * 2, tile + blk * RPI * HD);
  }
}

// Stages ROWS x HD bf16 rows of a matrix whose rows lie `rs` elements apart (packed [T, heads, HD]
// token rows: rs = heads * HD) into an LDS tile with swizzle SWZ. `src` is the tile's first row;
// only the first n_valid rows are read (the resource ends at the last of them), the others read as
// zero. Called by all NWAVES waves of the workgroup, as stage_tile.
template <int HD, int ROWS, int NWAVES, int (*SWZ)(int)>
__device__ __forceinline__ void stage_rows(const bf16* __restrict__ src, int rs, int n_valid, bf16* tile, int w,
                                           int lane) {
  constexpr int CH = HD / 8;
  constexpr int RPI = 1024 / (HD * 2);
  constexpr int BLOCKS = ROWS / RPI;
  static_assert(BLOCKS % NWAVES == 0, "tile geometry");
  const u32x4 rsrc = dma_rsrc(src, n_valid > 0 ? (min(n_valid, ROWS) - 1) * rs * 2 + HD * 2 : 0);
#pragma unroll
  for (int u = 0; u < BLOCKS / NWAVES; ++u) {
    const int blk = u * NWAVES + w;
    const int row = blk * RPI + lane / CH;
    load_to_lds<16>(rsrc, (row * rs + (((lane % CH) ^ SWZ(row)) * 8)) * 2, tile + blk * RPI * HD);
  }
}

// Address of the 16-byte chunk `chunk` of row `row` in a tile with swizzle SWZ.
template <int HD, int (*SWZ)(int)>
__device__ __forceinline__ const bf16* tile_chunk(const bf16* tile, int row, int chunk) {
  return tile + row * HD + ((chunk ^ SWZ(row)) * 8);
}

}  // namespace ra
