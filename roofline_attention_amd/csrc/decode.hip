// Split-KV decode attention for one query token per (sequence, head) over a bf16 KV cache.
//
// Decode is memory-bound at I = 2g/s FLOP/byte for group size g ("Why Fast GPUs Still Wait for
// Memory", section "Attention III - KV cache, GQA, MLA"), so the kernel is built to stream K and V
// at HBM rate: every K/V byte is read once, and all g query heads of a KV head are served from
// the same bytes (the grouped physical path, no K/V expansion). The key axis is split across
// workgroups in equal shares of all the keys of the batch, so ragged sequence lengths never leave
// a long serial tail; the partial (max, sum, output) triples are merged by a second kernel ("M4.2 -
// GPU Execution Model for Transformer Kernels", section 0x08: split-K trades parallelism for an
// extra reduction pass).
//
// Split kernel, persistent: two 4-wave workgroups per CU, each taking an equal contiguous share of
//   the batch's 32-key tiles laid end to end (stream-K); a share that spans several (sequence, KV
//   head) segments is processed one piece per segment. Within a piece each wave streams its
//   quarter of the tiles, held in registers (two tiles in flight), S^T and O^T on 16x16x32 bf16
//   MFMAs, and the waves' partial (max, sum, output) triples are merged in LDS into the piece's
//   record {m, l, np, -, o[d]} per query head, m in log2 units of the scaled score, o not yet
//   divided by l, np the number of pieces (records) of the segment (an int in a float's bits).
// Combine kernel, one wave per (query head, sequence): over the pieces j of its segment,
//   M = max m_j, L = sum 2^(m_j - M) l_j, O = sum 2^(m_j - M) o_j / L, LSE = ln 2 * (M + log2 L).
#include <math.h>

#include <algorithm>
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
std::atomic<int> g_cus[kMaxDevices];            // per device: compute units, once known

// Compute units of the current device (cached per device).
hipError_t device_cus(int* cus) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev >= 0 && dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return hipSuccess;
    }
  }
  int c = 0;
  err = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if (c < 1) c = 1;
  if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return hipSuccess;
}


constexpr int DEC_WAVES = 4;                             // waves per workgroup
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

// Per piece, wave w takes its quarter of the piece's tiles and works independently of the other
// waves until the merge. Decode moves bytes, so the kernel is organised around keeping enough of them
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
// taken in chunks of up to 16 query heads, each chunk a segment of its own (for grp > 16 each
// chunk reads the KV head's rows again).
constexpr int kDecodeAnyGroup = 16;

// Stream-K partition of the keys. Every (sequence b, KV head, head chunk) segment is that
// sequence's keys cut into 32-key tiles (units); the segments lie end to end (sequence-major, then
// KV head, then head chunk), U units in all. Workgroup w of P' = min(P, max(1, U / 32)) takes the
// units [floor(w U / P'), floor((w + 1) U / P')), at least 32 of them (1024 keys) when U >= 32:
// every workgroup streams the same number of bytes whatever the mix of lengths, the grid is one
// round of resident workgroups with one start-up each, and no slot waits for the dispatcher
// (measured with one workgroup per 1024-key split of each sequence: CUs held on average 1.5 of
// their 2 workgroup slots, and a freed slot waited a median 4.6 us for its next workgroup). A
// segment of u units meets at most ceil(u / 32) + 1 <= ceil(N_cap / 1024) + 1 workgroup ranges,
// each of which leaves one partial record. Every wave computes the partition from the lengths (one
// 4-byte load per lane and sequence); every result is wave-uniform.
struct DecodePart {
  long long U;  // units in all
  int P;        // workgroups that take a range (0 when U == 0)
  __device__ long long lo(int w) const { return (long long)w * U / P; }
  // workgroup whose range holds unit x
  __device__ int owner(long long x) const { return (int)(((x + 1) * P - 1) / U); }
};

__device__ __forceinline__ int units_of(const int32_t* __restrict__ kv_len, int b, int B, int N_cap) {
  return b < B ? (clamp_len(kv_len, b, N_cap) + DEC_TILE - 1) / DEC_TILE : 0;
}

__device__ __forceinline__ long long wave_sum_ll(long long x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ long long uniform_ll(long long x) {
  const uint64_t u = (uint64_t)x;
  return (long long)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32)) << 32) |
                     (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u));
}

__device__ __forceinline__ DecodePart decode_partition(const int32_t* __restrict__ kv_len, int B, int N_cap, int Hs,
                                                       int P) {
  const int lane = threadIdx.x & 63;
  long long tot = 0;
  for (int b0 = 0; b0 < B; b0 += 64) tot += wave_sum_ll(units_of(kv_len, b0 + lane, B, N_cap));
  DecodePart p;
  p.U = uniform_ll(tot * Hs);
  p.P = p.U == 0 ? 0 : (int)min((long long)P, max(1LL, p.U / (kDecodeSplit / DEC_TILE)));
  return p;
}

// The segment that holds unit x (x < U): sequence, segment index within the sequence
// (KV head * n_chunk + head chunk), its first unit and its unit count.
struct DecodeSeg {
  int b, s_in_b, u;
  long long start;
};
__device__ __forceinline__ DecodeSeg decode_segment(const int32_t* __restrict__ kv_len, int B, int N_cap, int Hs,
                                                    long long x) {
  const int lane = threadIdx.x & 63;
  long long base = 0;
  DecodeSeg sg{0, 0, 1, 0};
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int u = units_of(kv_len, b0 + lane, B, N_cap);
    const long long sz = (long long)u * Hs;
    long long incl = sz;  // inclusive prefix over the lanes
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    const long long excl = base + incl - sz;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(sz > 0 && excl <= x && x < excl + sz);
    if (hit != 0) {
      const int l = (int)__builtin_ctzll(hit);  // the one lane whose range holds x
      sg.b = b0 + l;
      sg.u = __builtin_amdgcn_readfirstlane(__shfl(u, l, 64));
      const long long e = uniform_ll(__shfl(excl, l, 64));
      sg.s_in_b = (int)((x - e) / sg.u);
      sg.start = e + (long long)sg.s_in_b * sg.u;
      return sg;
    }
    base += uniform_ll(__shfl(incl, 63, 64));
  }
  return sg;  // not reached for x < U
}

template <int HD, int G, bool PAGED>
__global__ __launch_bounds__(DEC_WAVES * 64, 2) void decode_split_kernel(
    const bf16* __restrict__ Qd, const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
    const int32_t* __restrict__ kv_len, float* __restrict__ ws, int B, int H, int H_kv, int N_cap, int n_rec,
    int P, float scale_log2, const int32_t* __restrict__ block_table, int max_pages, int page_shift,
    int num_pages, int grp, int n_chunk) {
  constexpr int CH = HD / 8;        // 16-byte chunks per row
  constexpr int KSTEPS = HD / 32;   // 16x16x32 k-steps over d
  constexpr int CB = HD / 16;       // 16-row blocks of O^T
  constexpr int VROWS = 64 / CH;    // V rows per wave load instruction
  constexpr int VLOADS = DEC_TILE / VROWS;
  constexpr int REC = HD + 4;
  constexpr int PER = HD / 64;
  static_assert(G <= 16, "query heads per workgroup");
  __shared__ bf16 vtile[DEC_WAVES][DEC_TILE * HD];
  __shared__ DecodeMerge<HD, G> mg;

  constexpr bool ANY = G == kDecodeAnyGroup;
  const int Hs = H_kv * n_chunk;  // segments per sequence
  const DecodePart part = decode_partition(kv_len, B, N_cap, Hs, P);
  const int wg = blockIdx.x;
  if (wg >= part.P) return;  // uniform over the workgroup, before any barrier

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;  // MFMA column = query head head0 + col (valid when < gh)
  const int q4 = lane >> 4;   // 16-lane group
  bf16* vt = vtile[w];
  // K A-operand of half h, k-step kk: row 16h + col, bytes (32kk + 8q4) * 2 of the row.
  const int k_off = col * HD * 2 + q4 * 16;
  // V rows: lane holds chunk (lane % CH) of row (lane / CH) + VROWS * i.
  const int v_off = (lane / CH) * HD * 2 + (lane % CH) * 16;
  // V^T A-operand (transposed read): in 16-lane group q4, source lane 4e + j points at key row
  // base + 4*q4 + e and column 16cb + 4j; the lane receives column 16cb + col of 4 keys. The LDS
  // tile stores chunk c of row r at position c ^ (2r mod CH): the 8 rows x 2 chunks a 32-lane
  // read touches fall in distinct banks.
  const int v_e = (lane & 15) >> 2;
  const int v_j = lane & 3;
  const int st_row = lane / CH;
  const float c = scale_log2;

  // The workgroup's units, one piece per segment they touch (usually one or two): within a piece
  // wave w takes units [n w / 4, n (w + 1) / 4) of its n, and the four waves' results merge into
  // the piece's record, slot (this workgroup - the segment's first workgroup).
  const long long x_end = part.lo(wg + 1);
  for (long long xu = part.lo(wg); xu < x_end;) {
    const DecodeSeg sg = decode_segment(kv_len, B, N_cap, Hs, xu);
    const long long p_end = min(x_end, sg.start + sg.u);
    const int seg_w0 = part.owner(sg.start);
    const int slot = wg - seg_w0;
    const int n_pieces = part.owner(sg.start + sg.u - 1) - seg_w0 + 1;  // records of this segment
    const int b = sg.b;
    const int hk = sg.s_in_b / n_chunk;
    const int chunk = sg.s_in_b % n_chunk;
    const int gsize = ANY ? grp : G;                        // query heads per KV head
    const int head0 = hk * gsize + 16 * chunk;              // first query head of this piece
    const int gh = ANY ? min(16, gsize - 16 * chunk) : G;   // query heads of this piece
    const int len = clamp_len(kv_len, b, N_cap);
    const int n = (int)(p_end - xu);
    const int first = (int)(xu - sg.start);
    const int kw_begin = (first + n * w / DEC_WAVES) * DEC_TILE;  // this wave's first key
    const int n_keys = max(min(len, (first + n * (w + 1) / DEC_WAVES) * DEC_TILE) - kw_begin, 0);
    const int n_tiles = (n_keys + DEC_TILE - 1) / DEC_TILE;

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

    f32x4 acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;

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
    for (int hq = w; hq < gh; hq += DEC_WAVES) {
      float M = mg.m[0][hq];
#pragma unroll
      for (int v = 1; v < DEC_WAVES; ++v) M = fmaxf(M, mg.m[v][hq]);  // finite: some wave has keys
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
      float* rec = ws + (((size_t)b * H + head0 + hq) * n_rec + slot) * REC;
      if (lane == 0) {
        rec[0] = M;
        rec[1] = L;
        rec[2] = __int_as_float(n_pieces);
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) rec[4 + lane * PER + e] = o[e];
    }
    __syncthreads();  // the merge tiles are reused by the next piece
    xu = p_end;
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

constexpr int kFastRecs = 16;  // record counts the combine merges with one round of loads

// Merge of the partial records of one (sequence, query head): the pieces of its segment, one per
// workgroup share the segment meets, in record slots 0 .. np - 1; the split kernel stores np in the
// third field of every piece's record (slot 0's is read). M, the weights 2^(m_j - M) and L take one
// round of parallel loads and wave reductions; the output then sums the partial rows with
// independent loads, PER elements per lane.
template <int HD>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ ws,
                                                            const int32_t* __restrict__ kv_len,
                                                            bf16* __restrict__ Od, float* __restrict__ lse,
                                                            int H, int N_cap, int n_rec) {
  constexpr int REC = HD + 4;
  constexpr int PER = HD / 64;  // output elements per lane
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  bf16* out = Od + ((size_t)b * H + h) * HD;
  const float* recs = ws + ((size_t)b * H + h) * n_rec * REC;
  const int len = clamp_len(kv_len, b, N_cap);
  if (n_rec <= kFastRecs) {
    // Up to kFastRecs slots (caches of up to 15 * 1024 rows): every record load is issued at once,
    // beside the length load, so the merge costs one memory round trip. Slots at or past the
    // segment's np lie inside the workspace but were not written by this call; selects, not zero
    // weights, keep them out (they may hold anything, NaN included).
    float4 hd = make_float4(-INFINITY, 0.f, 0.f, 0.f);
    if (lane < n_rec) hd = *reinterpret_cast<const float4*>(recs + (size_t)lane * REC);
    float v[kFastRecs][PER];
#pragma unroll
    for (int j = 0; j < kFastRecs; ++j) {
      if (j < n_rec) {
#pragma unroll
        for (int e = 0; e < PER; ++e) v[j][e] = recs[(size_t)j * REC + 4 + lane * PER + e];
      }
    }
    if (len == 0) {
#pragma unroll
      for (int e = 0; e < PER; ++e) out[lane * PER + e] = to_bf16(0.f);
      if (lse != nullptr && lane == 0) lse[(size_t)b * H + h] = -INFINITY;
      return;
    }
    const int np = __builtin_amdgcn_readfirstlane(__float_as_int(__shfl(hd.z, 0, 64)));  // slot 0's count
    const bool mine = lane < np;
    const float m = mine ? hd.x : -INFINITY;
    const float M = wave_max(m);  // finite: every piece holds at least one key
    const float wgt = mine ? fast_exp2(m - M) : 0.f;
    const float L = wave_sum(mine ? wgt * hd.y : 0.f);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < kFastRecs; ++j) {
      if (j < np) {  // uniform over the wave
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
  if (len == 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) out[lane * PER + e] = to_bf16(0.f);
    if (lse != nullptr && lane == 0) lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  const int np = __float_as_int(recs[2]);  // slot 0's count (<= n_rec)
  auto ml_of = [&](int s) {
    return s < np ? *reinterpret_cast<const float2*>(recs + (size_t)s * REC) : make_float2(-INFINITY, 0.f);
  };
  const float2 ml0 = ml_of(lane);
  float M = ml0.x;
  for (int s = lane + 64; s < np; s += 64) M = fmaxf(M, recs[(size_t)s * REC]);
  M = wave_max(M);  // finite: every piece holds at least one key
  float L = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < np; s0 += 64) {
    const float2 ml = s0 == 0 ? ml0 : ml_of(s0 + lane);
    const float wgt = fast_exp2(ml.x - M);  // 0 past np
    L = fmaf(wgt, ml.y, L);
    const int cnt = min(64, np - s0);
    // Four records per step, loads issued together; steps past cnt re-read the last valid
    // record with weight 0.
    for (int j0 = 0; j0 < cnt; j0 += 4) {
      float wj[4], vv[4][PER];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = min(j0 + q, cnt - 1);
        wj[q] = j0 + q < cnt ? __shfl(wgt, j, 64) : 0.f;
        const float* r = recs + (size_t)(s0 + j) * REC + 4 + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) vv[q][e] = r[e];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(wj[q], vv[q][e], acc[e]);
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
  const int n_rec = n_split + 1;  // record slots per (sequence, query head)
  const int grp = H / H_kv;
  const int n_chunk = G == kDecodeAnyGroup ? (grp + 15) / 16 : 1;
  int cus = 0;
  hipError_t err = device_cus(&cus);
  if (err != hipSuccess) return err;
  // Two resident workgroups per CU (the kernel's register budget), never more than the partition
  // can use (each range holds at least kDecodeSplit keys).
  const int P = (int)std::min<long long>(2LL * cus, (long long)B * H_kv * n_chunk * n_split);
  {
    TimedScope ts(split_name, stream);
    hipLaunchKernelGGL((decode_split_kernel<HD, G, PAGED>), dim3(P), dim3(DEC_WAVES * 64), 0, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(kc), static_cast<const bf16*>(vc),
                       kv_len, static_cast<float*>(ws), B, H, H_kv, N_cap, n_rec, P, scale * kLog2e, block_table,
                       max_pages, page_shift, num_pages, grp, n_chunk);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    TimedScope ts(combine_name, stream);
    hipLaunchKernelGGL((decode_combine_kernel<HD>), dim3(H, B), dim3(64), 0, stream,
                       static_cast<const float*>(ws), kv_len, static_cast<bf16*>(o), lse, H, N_cap, n_rec);
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
  const size_t n_rec = ((size_t)N_cap + kDecodeSplit - 1) / kDecodeSplit + 1;
  return (size_t)B * H * n_rec * (size_t)(d + 4) * sizeof(float);
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
