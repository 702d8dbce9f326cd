// Split-KV decode attention for one query token per (sequence, head) over a bf16 KV cache.
//
// Decode is memory-bound at I = 2g/s FLOP/byte for group size g ("Why Fast GPUs Still Wait for
// Memory", section "Attention III - KV cache, GQA, MLA"), so the kernel is built to stream K and V
// at HBM rate: every K/V byte is read once, and all g query heads of a KV head are served from
// the same bytes (the grouped physical path, no K/V expansion). The key axis is split into
// fixed-size chunks, one workgroup each, so ragged sequence lengths never leave a long serial tail;
// the partial (max, sum, output) triples are merged by a second kernel ("M4.2 - GPU Execution
// Model for Transformer Kernels", section 0x08: split-K trades parallelism for an extra
// reduction pass).
//
// Split kernel, one 4-wave workgroup per (sequence, KV head, 1024-key split), launched split-major
//   so the 8 XCDs share every split evenly; each wave streams 256 keys in 32-key tiles held in
//   registers (two tiles in flight), S^T and O^T on 16x16x32 bf16 MFMAs, and the waves' partial
//   (max, sum, output) triples are merged in LDS. The record of each query head and split is
//   {m, l, -, -, o[d]} with m in log2 units of the scaled score and o not yet divided by l.
// Combine kernel, one wave per (query head, sequence): M = max m_s, L = sum 2^(m_s - M) l_s,
//   O = sum 2^(m_s - M) o_s / L, LSE = ln 2 * (M + log2 L).
#include <math.h>

#include <atomic>

#include "../../include/attn.h"
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace ra {
namespace {

// Split-record scratch of attn_decode_noalloc, for callers that cannot allocate: one copy per GPU
// the library runs on, held until the process ends. In host code this name is only a stand-in for
// the symbol; kernels receive the device address that hipGetSymbolAddress returns
// (decode_scratch_address below), never the name itself. The records need no initial contents.
static __device__ __align__(256) unsigned char scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];  // per device: scratch's device address, once known


constexpr int DEC_WAVES = 4;                             // waves per workgroup
constexpr int DEC_WAVE_KEYS = kDecodeSplit / DEC_WAVES;  // keys per wave (256)
constexpr int DEC_TILE = 32;                             // keys per tile

__device__ __forceinline__ int clamp_len(const int32_t* kv_len, int b, int N_cap) {
  const int len = kv_len[b];
  return len < 0 ? 0 : (len > N_cap ? N_cap : len);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// K/V bytes are read exactly once: loads carry the non-temporal cache policy (gfx950 cache-policy
// bit 1, "nt"), which keeps the stream from displacing other lines; measured 10% faster here.
__device__ __forceinline__ bf16x8 buffer_load16_nt(__amdgpu_buffer_rsrc_t rsrc, int voffset) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voffset, 0, 2));
}

// Buffer resource over [base, base + bytes) whose inputs are wave-uniform by construction; the
// readfirstlanes tell the compiler so, which keeps the descriptor in scalar registers (otherwise
// a descriptor built from loaded values is treated as divergent and every load is wrapped in a
// loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  // readfirstlane returns int: each half goes through uint32_t before widening, or the low half
  // would be sign-extended into the high one.
  const uint64_t ua = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  return make_rsrc((const void*)(uintptr_t)ua, __builtin_amdgcn_readfirstlane(bytes));
}

template <int HD, int G>
struct DecodeMerge {
  float m[DEC_WAVES][G];
  float l[DEC_WAVES][G];
  float o[DEC_WAVES][G][HD];
};

// One workgroup = 4 waves over kDecodeSplit consecutive keys of one (sequence, KV head); wave w
// takes keys [256w, 256w + 256) of the split and works independently of the other waves until
// the final merge. Decode moves bytes, so the kernel is organised around keeping enough of them
// in flight: by Little's law the HBM rate needs roughly rate x latency bytes outstanding, more
// than the LDS can buffer, so each wave stages its 32-key K/V tiles in registers, two tiles in
// flight (the register file is several times larger than the LDS). Per tile:
//   S^T = K Q^T on 16x16x32 MFMAs, the K rows used directly from registers as the A operand
//   (16 keys x 32 d), Q^T as the B operand (the g query heads as columns, zero-padded to 16);
//   online softmax per head on the few lanes that hold real heads;
//   V written to the wave's LDS tile and read back transposed as the A operand of
//   O^T += V^T P^T (16x16x32 MFMAs).
// Register loads of tiles past the wave's last key return zeros (buffer range check).
// PAGED: the caches are pages [num_pages, H_kv, 2^page_shift, d] and row j of sequence b lives in
// page block_table[b * max_pages + j >> page_shift]; a 32-key tile never straddles a page (pages
// hold a multiple of 32 rows), so each tile is one contiguous run read through its own buffer
// resource. Page ids are looked up two tiles ahead of their loads and clamped into
// [0, num_pages), so a malformed table cannot send a load outside the caches.
// G = 1, 2, 4 or 8: the group size, exactly. G = kDecodeAnyGroup: any group size `grp` (= H / H_kv),
// taken in chunks of up to 16 query heads, one workgroup per chunk (for grp > 16 each chunk reads
// the KV head's rows again).
constexpr int kDecodeAnyGroup = 16;

// Work items of the split kernel: (split s, sequence b, KV head hk) for every split that holds keys,
// enumerated split-major (split 0 of every sequence and KV head, then split 1, ...). Workgroup
// `lin` in launch order takes item lin / n_chunk (n_chunk workgroups per item), and ids past the
// last item exit. The workgroups that own no keys thus come after every working one in launch
// order: spread among them, as they were with one workgroup per (split, sequence, KV head), each
// held a dispatch slot while it read its length and exited, and freed CU slots sat empty for
// microseconds (measured: a CU held on average 1.43 of its 2 workgroup slots over the kernel).
// Computed by every wave from the lengths (one 4-byte load per lane and sequence); all results
// are wave-uniform.
struct DecodeItem {
  int split, b, hk, len;
};
__device__ __forceinline__ bool decode_item(const int32_t* __restrict__ kv_len, int B, int H_kv, int N_cap,
                                            int n_split, int item, DecodeItem& out) {
  const int lane = threadIdx.x & 63;
  auto n_splits_of = [&](int b) { return b < B ? (clamp_len(kv_len, b, N_cap) + kDecodeSplit - 1) / kDecodeSplit : 0; };
  const int ns0 = n_splits_of(lane);  // the common case, B <= 64, needs no other load
  int rem = item;
  for (int s = 0; s < n_split; ++s) {
    int cnt = 0;  // sequences with more than s splits
    for (int b0 = 0; b0 < B; b0 += 64) {
      const int ns = b0 == 0 ? ns0 : n_splits_of(b0 + lane);
      cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(ns > s));
    }
    if (rem < cnt * H_kv) {
      const int j = rem / H_kv;  // the j-th such sequence, in order
      int seen = 0;
      for (int b0 = 0; b0 < B; b0 += 64) {
        const int ns = b0 == 0 ? ns0 : n_splits_of(b0 + lane);
        const uint64_t mask = __builtin_amdgcn_ballot_w64(ns > s);
        const int c = __builtin_popcountll(mask);
        if (j < seen + c) {
          // lane whose bit is set with exactly j - seen set bits below it
          const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
          const uint64_t hit = __builtin_amdgcn_ballot_w64(ns > s && below == j - seen);
          const int b = b0 + (int)__builtin_ctzll(hit);
          out.split = s;
          out.b = b;
          out.hk = rem % H_kv;
          out.len = clamp_len(kv_len, b, N_cap);
          return true;
        }
        seen += c;
      }
    }
    rem -= cnt * H_kv;
  }
  return false;
}

template <int HD, int G, bool PAGED>
__global__ __launch_bounds__(DEC_WAVES * 64, 2) void decode_split_kernel(
    const bf16* __restrict__ Qd, const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
    const int32_t* __restrict__ kv_len, float* __restrict__ ws, int H, int H_kv, int N_cap,
    int n_split, float scale_log2, const int32_t* __restrict__ block_table, int max_pages, int page_shift,
    int num_pages, int grp, int n_chunk) {
  constexpr int CH = HD / 8;        // 16-byte chunks per row
  constexpr int KSTEPS = HD / 32;   // 16x16x32 k-steps over d
  constexpr int CB = HD / 16;       // 16-row blocks of O^T
  constexpr int VROWS = 64 / CH;    // V rows per wave load instruction
  constexpr int VLOADS = DEC_TILE / VROWS;
  constexpr int REC = HD + 4;
  static_assert(G <= 16, "query heads per workgroup");
  __shared__ bf16 vtile[DEC_WAVES][DEC_TILE * HD];
  __shared__ DecodeMerge<HD, G> mg;

  // Grid (B * H_kv * n_chunk, n_split) in launch order (x fastest): workgroups reach the 8 XCDs
  // round-robin, so consecutive ids walk the (sequence, KV head, head chunk) triples of one split
  // and every XCD gets an even share of each split. (With the split index fastest, split s would
  // always land on XCD s mod 8 and short sequences would load only the first few XCDs.)
  constexpr bool ANY = G == kDecodeAnyGroup;
  const int lin = (int)blockIdx.y * (int)gridDim.x + (int)blockIdx.x;
  const int chunk = ANY ? lin % n_chunk : 0;
  DecodeItem it;
  if (!decode_item(kv_len, (int)gridDim.x / (H_kv * n_chunk), H_kv, N_cap, n_split, ANY ? lin / n_chunk : lin, it))
    return;  // uniform over the workgroup, before any barrier
  const int split = it.split;
  const int hk = it.hk;
  const int b = it.b;
  const int gsize = ANY ? grp : G;                                // query heads per KV head
  const int head0 = hk * gsize + 16 * chunk;                      // first query head of this workgroup
  const int gh = ANY ? min(16, gsize - 16 * chunk) : G;           // query heads of this workgroup
  const int len = it.len;
  const int k_begin = split * kDecodeSplit;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;  // MFMA column = query head head0 + col (valid when < gh)
  const int q4 = lane >> 4;   // 16-lane group
  const int kw_begin = k_begin + w * DEC_WAVE_KEYS;
  const int kw_end = min(len, kw_begin + DEC_WAVE_KEYS);
  const int n_keys = max(kw_end - kw_begin, 0);
  const int n_tiles = (n_keys + DEC_TILE - 1) / DEC_TILE;
  bf16* vt = vtile[w];

  // Q^T as the B operand: column col = head head0 + col, k-group q4 holds d = 32kk + 8q4 .. +7.
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    qf[kk] = col < gh ? *reinterpret_cast<const bf16x8*>(Qd + ((size_t)b * H + head0 + col) * HD + 32 * kk + 8 * q4)
                      : bf16x8{};
  }

  const size_t head = PAGED ? 0 : ((size_t)b * H_kv + hk) * (size_t)N_cap * HD;
  const auto krs = make_rsrc(Kc + head + (size_t)kw_begin * HD, PAGED ? 0 : n_keys * HD * 2);
  const auto vrs = make_rsrc(Vc + head + (size_t)kw_begin * HD, PAGED ? 0 : n_keys * HD * 2);
  // K A-operand of half h, k-step kk: row 16h + col, bytes (32kk + 8q4) * 2 of the row.
  const int k_off = col * HD * 2 + q4 * 16;
  // V rows: lane holds chunk (lane % CH) of row (lane / CH) + VROWS * i.
  const int v_off = (lane / CH) * HD * 2 + (lane % CH) * 16;

  struct Tile {
    bf16x8 k[2][KSTEPS];
    bf16x8 v[VLOADS];
  };
  // Physical page of tile t (PAGED only): the table entry is clamped to the table row, the id
  // into [0, num_pages).
  auto lookup = [&](int t) {
    if constexpr (PAGED) {
      const int j = min((kw_begin + t * DEC_TILE) >> page_shift, max_pages - 1);
      // Same address in every lane: readfirstlane keeps the id (and the tile's buffer resource
      // built from it) in scalar registers.
      return __builtin_amdgcn_readfirstlane(min(max(block_table[(size_t)b * max_pages + j], 0), num_pages - 1));
    } else {
      return 0;
    }
  };
  auto load = [&](int t, Tile& tl, int pid) {
    int base = t * DEC_TILE * HD * 2;
    auto kr = krs, vr = vrs;
    if constexpr (PAGED) {
      const int off = (kw_begin + t * DEC_TILE) & ((1 << page_shift) - 1);
      const size_t row = (((size_t)pid * H_kv + hk) << page_shift) + off;
      const int bytes = min(max(n_keys - t * DEC_TILE, 0), DEC_TILE) * HD * 2;  // 0 past the wave's keys
      kr = uniform_rsrc(Kc + row * HD, bytes);
      vr = uniform_rsrc(Vc + row * HD, bytes);
      base = 0;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) tl.k[h][kk] = buffer_load16_nt(kr, base + k_off + h * 16 * HD * 2 + kk * 64);
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) tl.v[i] = buffer_load16_nt(vr, base + v_off + i * VROWS * HD * 2);
  };

  // V^T A-operand (transposed read): in 16-lane group q4, source lane 4e + j points at key row
  // base + 4*q4 + e and column 16cb + 4j; the lane receives column 16cb + col of 4 keys. The LDS
  // tile stores chunk c of row r at position c ^ (2r mod CH): the 8 rows x 2 chunks a 32-lane
  // read touches fall in distinct banks.
  const int v_e = (lane & 15) >> 2;
  const int v_j = lane & 3;
  const int st_row = lane / CH;

  f32x4 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = scale_log2;

  auto consume = [&](int t, const Tile& tl) {
    // V tile to LDS (swizzled), consumed below by this wave only.
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int row = i * VROWS + st_row;
      *reinterpret_cast<bf16x8*>(vt + row * HD + (((lane % CH) ^ ((2 * row) & (CH - 1))) * 8)) = tl.v[i];
    }
    // S^T for keys 16*half + 4*q4 + r (r = 0..3), column = head.
    f32x4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x4{};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) s[h] = mfma16(tl.k[h][kk], qf[kk], s[h]);
    }
    const int key0 = t * DEC_TILE;  // relative to kw_begin
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 16 * h + 4 * q4 + r;
        const float v = key < n_keys ? s[h][r] * c : -INFINITY;
        x[4 * h + r] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // Tile 0 holds the wave's first key, so m_run is finite after it; a fully masked tile
    // later gives alpha = 1 and p = 0.
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    // The normaliser sums the bf16-rounded probabilities, the values that multiply V.
    bf16x8 pb;
    float tsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pb[e] = to_bf16(fast_exp2(x[e] - m_new));
      tsum += to_f32(pb[e]);
    }
    l_run = fmaf(l_run, alpha, tsum);
    // Unconditional rescale: a branch here would split the loop body, and the compiler would
    // then sink the next tile's loads past it and serialise them behind the current tile.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
    // O^T += V^T P^T: k-slot e < 4 is key 4*q4 + e, e >= 4 is key 16 + 4*q4 + (e - 4).
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int r0 = 4 * q4 + v_e;
      const int r1 = 16 + 4 * q4 + v_e;
      const bf16* p0 = vt + r0 * HD + (((2 * cb + (v_j >> 1)) ^ ((2 * r0) & (CH - 1))) * 8) + 4 * (v_j & 1);
      const bf16* p1 = vt + r1 * HD + (((2 * cb + (v_j >> 1)) ^ ((2 * r1) & (CH - 1))) * 8) + 4 * (v_j & 1);
      acc[cb] = mfma16(__builtin_shufflevector(lds_read_tr(p0), lds_read_tr(p1), 0, 1, 2, 3, 4, 5, 6, 7), pb, acc[cb]);
    }
  };

  // Two tiles in flight: the loads of tile t + 2 are issued as soon as tile t is consumed. The
  // loop body is one basic block over a pair of tiles, and the loads are unconditional (tiles
  // past the wave's keys read as zeros, and a whole tile past the end is fully masked, which
  // leaves m, l and O unchanged), so the wait before each consume covers only the tile it needs.
  {
    Tile ta, tb;
    load(0, ta, lookup(0));
    load(1, tb, lookup(1));
    int pa = lookup(2), pb = lookup(3);  // page ids two tiles ahead of their loads
    for (int t = 0; t < n_tiles; t += 2) {
      consume(t, ta);
      load(t + 2, ta, pa);
      pa = lookup(t + 4);
      consume(t + 1, tb);
      load(t + 3, tb, pb);
      pb = lookup(t + 5);
    }
  }

  // l: each lane summed its 8 keys per tile; the 4 lanes of a head column hold the rest.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  if (col < gh) {
    if (q4 == 0) {
      mg.m[w][col] = m_run;  // -inf for a wave with no keys
      mg.l[w][col] = l_run;
    }
    // O^T rows c = 16cb + 4*q4 + r of head column col.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) *reinterpret_cast<f32x4*>(&mg.o[w][col][16 * cb + 4 * q4]) = acc[cb];
  }
  __syncthreads();
  constexpr int PER = HD / 64;
  for (int hq = w; hq < gh; hq += DEC_WAVES) {
    float M = mg.m[0][hq];  // wave 0 always has keys
#pragma unroll
    for (int v = 1; v < DEC_WAVES; ++v) M = fmaxf(M, mg.m[v][hq]);
    float L = 0.f, o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
    for (int v = 0; v < DEC_WAVES; ++v) {
      const float wgt = fast_exp2(mg.m[v][hq] - M);  // 0 for a wave with no keys
      L = fmaf(wgt, mg.l[v][hq], L);
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = fmaf(wgt, mg.o[v][hq][lane * PER + e], o[e]);
    }
    float* rec = ws + (((size_t)b * H + head0 + hq) * n_split + split) * REC;
    if (lane == 0) {
      rec[0] = M;
      rec[1] = L;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) rec[4 + lane * PER + e] = o[e];
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

constexpr int kFastSplits = 8;  // split counts the combine merges with one round of loads

// One wave per (query head, sequence). Lane s holds (m, l) of split s (64 splits per pass), so
// M, the weights 2^(m_s - M) and L take one round of parallel loads and wave reductions; the
// output then sums the splits' partial rows with independent loads, PER elements per lane.
template <int HD>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws,
                                                            const int32_t* __restrict__ kv_len,
                                                            bf16* __restrict__ Od, float* __restrict__ lse,
                                                            int H, int N_cap, int n_split) {
  constexpr int REC = HD + 4;
  constexpr int PER = HD / 64;  // output elements per lane
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  bf16* out = Od + ((size_t)b * H + h) * HD;
  const float* recs = ws + ((size_t)b * H + h) * n_split * REC;
  if (n_split <= kFastSplits) {
    // Up to kFastSplits splits (caches of up to 8192 rows): every record load is issued at once,
    // beside the length load, so the merge costs one memory round trip instead of three (length,
    // then maxima, then partial rows). Records of splits at or past the sequence's last one lie
    // inside the workspace but were not written by this call; selects, not zero weights, keep them
    // out (they may hold anything, NaN included).
    float2 ml = make_float2(-INFINITY, 0.f);
    if (lane < n_split) ml = *reinterpret_cast<const float2*>(recs + (size_t)lane * REC);
    float v[kFastSplits][PER];
#pragma unroll
    for (int j = 0; j < kFastSplits; ++j) {
      if (j < n_split) {
#pragma unroll
        for (int e = 0; e < PER; ++e) v[j][e] = recs[(size_t)j * REC + 4 + lane * PER + e];
      }
    }
    const int len = clamp_len(kv_len, b, N_cap);
    const int ns = (len + kDecodeSplit - 1) / kDecodeSplit;
    if (ns == 0) {
#pragma unroll
      for (int e = 0; e < PER; ++e) out[lane * PER + e] = to_bf16(0.f);
      if (lse != nullptr && lane == 0) lse[(size_t)b * H + h] = -INFINITY;
      return;
    }
    const bool mine = lane < ns;
    const float m = mine ? ml.x : -INFINITY;
    const float M = wave_max(m);  // finite: every split below ns holds at least one key
    const float wgt = mine ? fast_exp2(m - M) : 0.f;
    const float L = wave_sum(mine ? wgt * ml.y : 0.f);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < kFastSplits; ++j) {
      if (j < ns) {  // uniform over the wave
        const float wj = __shfl(wgt, j, 64);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj, v[j][e], acc[e]);
      }
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < PER; ++e) out[lane * PER + e] = to_bf16(acc[e] * inv);
    if (lse != nullptr && lane == 0) lse[(size_t)b * H + h] = (M + log2f(L)) * kLn2;
    return;
  }
  const int len = clamp_len(kv_len, b, N_cap);
  const int ns = (len + kDecodeSplit - 1) / kDecodeSplit;
  if (ns == 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) out[lane * PER + e] = to_bf16(0.f);
    if (lse != nullptr && lane == 0) lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  auto ml_of = [&](int s) {
    return s < ns ? *reinterpret_cast<const float2*>(recs + (size_t)s * REC) : make_float2(-INFINITY, 0.f);
  };
  const float2 ml0 = ml_of(lane);
  float M = ml0.x;
  for (int s = lane + 64; s < ns; s += 64) M = fmaxf(M, recs[(size_t)s * REC]);
  M = wave_max(M);  // finite: every split below ns holds at least one key
  float L = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const float2 ml = s0 == 0 ? ml0 : ml_of(s0 + lane);
    const float wgt = fast_exp2(ml.x - M);  // 0 past ns
    L = fmaf(wgt, ml.y, L);
    const int cnt = min(64, ns - s0);
    // Four splits per step, loads issued together; steps past cnt re-read the last valid
    // record (the workspace beyond ns is never written) with weight 0.
    for (int j0 = 0; j0 < cnt; j0 += 4) {
      float wj[4], v[4][PER];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = min(j0 + u, cnt - 1);
        wj[u] = j0 + u < cnt ? __shfl(wgt, j, 64) : 0.f;
        const float* r = recs + (size_t)(s0 + j) * REC + 4 + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) v[u][e] = r[e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj[u], v[u][e], acc[e]);
    }
  }
  L = wave_sum(L);
  const float inv = 1.f / L;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[lane * PER + e] = to_bf16(acc[e] * inv);
  if (lse != nullptr && lane == 0) lse[(size_t)b * H + h] = (M + log2f(L)) * kLn2;
}

template <int HD, int G, bool PAGED>
hipError_t launch(const void* q, const void* kc, const void* vc, void* o, float* lse, const int32_t* kv_len,
                  int B, int H, int H_kv, int N_cap, float scale, void* ws, hipStream_t stream,
                  const char* split_name, const char* combine_name, const int32_t* block_table, int max_pages,
                  int page_shift, int num_pages) {
  const int n_split = (N_cap + kDecodeSplit - 1) / kDecodeSplit;
  const int grp = H / H_kv;
  const int n_chunk = G == kDecodeAnyGroup ? (grp + 15) / 16 : 1;
  {
    TimedScope ts(split_name, stream);
    hipLaunchKernelGGL((decode_split_kernel<HD, G, PAGED>), dim3(B * H_kv * n_chunk, n_split), dim3(DEC_WAVES * 64),
                       0, stream, static_cast<const bf16*>(q), static_cast<const bf16*>(kc),
                       static_cast<const bf16*>(vc), kv_len, static_cast<float*>(ws), H, H_kv, N_cap, n_split,
                       scale * kLog2e, block_table, max_pages, page_shift, num_pages, grp, n_chunk);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    TimedScope ts(combine_name, stream);
    hipLaunchKernelGGL((decode_combine_kernel<HD>), dim3(H, B), dim3(64), 0, stream,
                       static_cast<const float*>(ws), kv_len, static_cast<bf16*>(o), lse, H, N_cap, n_split);
  }
  return hipGetLastError();
}

// Paging descriptor of one call (block_table == nullptr: contiguous caches).
struct Pages {
  const int32_t* table;
  int max_pages, page_shift, num_pages;
};

template <int HD, bool PAGED>
hipError_t launch_g(int G, const void* q, const void* kc, const void* vc, void* o, float* lse,
                    const int32_t* kv_len, int B, int H, int H_kv, int N_cap, float scale, void* ws,
                    hipStream_t stream, const Pages& pg) {
  const char* comb = "decode_combine";
  switch (G) {
    case 1: return launch<HD, 1, PAGED>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                        PAGED ? "decode_paged_split_g1" : "decode_split_g1", comb, pg.table,
                                        pg.max_pages, pg.page_shift, pg.num_pages);
    case 2: return launch<HD, 2, PAGED>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                        PAGED ? "decode_paged_split_g2" : "decode_split_g2", comb, pg.table,
                                        pg.max_pages, pg.page_shift, pg.num_pages);
    case 4: return launch<HD, 4, PAGED>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                        PAGED ? "decode_paged_split_g4" : "decode_split_g4", comb, pg.table,
                                        pg.max_pages, pg.page_shift, pg.num_pages);
    case 8: return launch<HD, 8, PAGED>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                        PAGED ? "decode_paged_split_g8" : "decode_split_g8", comb, pg.table,
                                        pg.max_pages, pg.page_shift, pg.num_pages);
    default:
      return launch<HD, kDecodeAnyGroup, PAGED>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                                PAGED ? "decode_paged_split_any" : "decode_split_any", comb,
                                                pg.table, pg.max_pages, pg.page_shift, pg.num_pages);
  }
}

}  // namespace

size_t decode_workspace_bytes(int B, int H, int N_cap, int d) {
  const size_t n_split = ((size_t)N_cap + kDecodeSplit - 1) / kDecodeSplit;
  return (size_t)B * H * n_split * (size_t)(d + 4) * sizeof(float);
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, void* o, float* lse,
                         const int32_t* kv_len, int B, int H, int H_kv, int N_cap, int d, float scale,
                         void* ws, hipStream_t stream) {
  const int G = H / H_kv;
  const Pages none{nullptr, 1, 0, 1};
  return d == 128 ? launch_g<128, false>(G, q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream, none)
                  : launch_g<64, false>(G, q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream, none);
}

hipError_t decode_scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  void* p = cached ? g_scratch_ptr[dev].load(std::memory_order_acquire) : nullptr;
  if (p == nullptr) {
    // with the device current: each GPU holds its own copy of the array at its own address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    if (cached) g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse,
                               const int32_t* kv_len, const int32_t* block_table, int B, int H, int H_kv,
                               int num_pages, int page_size, int max_pages, int d, float scale, void* ws,
                               hipStream_t stream) {
  const int G = H / H_kv;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  const Pages pg{block_table, max_pages, shift, num_pages};
  const int N_cap = max_pages * page_size;
  return d == 128
             ? launch_g<128, true>(G, q, k_pages, v_pages, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream, pg)
             : launch_g<64, true>(G, q, k_pages, v_pages, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream, pg);
}

}  // namespace ra
