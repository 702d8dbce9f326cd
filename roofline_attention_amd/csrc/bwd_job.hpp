// Work of one workgroup of the attention backward on gfx950: the key-major dK/dV item and the
// query-major dQ item, as device functions shared by the backward kernels and the fused
// forward+backward kernel. The algorithm, tiling and MFMA layouts are described with the kernels
// in bwd.hip.
#pragma once

#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "lds_tile.hpp"

namespace ra {


constexpr int BWD_THREADS = 256;
// Waves per SIMD the register budget is sized for. At d = 128 the key-major kernel holds K, V
// operands and fp32 dK, dV accumulators (about 330 registers): one wave per SIMD keeps the
// accumulators in AGPRs without spilling, which measured faster than two spilling waves. At d = 64
// the same work fits two waves per SIMD (about 230 registers) and those run faster (below).
#ifndef RA_DKDV_WAVES_PER_SIMD
#define RA_DKDV_WAVES_PER_SIMD 1
#endif
template <int HD>
constexpr int dkdv_waves_per_simd() { return HD == 64 ? 2 : RA_DKDV_WAVES_PER_SIMD; }
#ifndef RA_DKDV_PAIR
#define RA_DKDV_PAIR 0
#endif
#ifndef RA_DQ_WAVES_PER_SIMD
#define RA_DQ_WAVES_PER_SIMD 2
#endif
constexpr int BWD_BQ = 64;   // queries per staged tile in the key-major kernel
constexpr int BWD_BK = 64;   // keys per staged tile in the query-major kernel


// Per-lane constants of the transposed read over a [rows][HD] tile with swizzle SWZ: in its
// 16-lane group, source lane 4e + j points at row (4g + e) of an 8-row-aligned block and element
// column 16 * ((lane / 16) % 2) + 4j of a 32-column block. The swizzle of that row depends on the
// block's row base only through its bit 3 (the second half of a 16-row k-step), so two lane
// constants cover both halves. Returns the element offset for (row base rb, column block cb).
template <int HD, int (*SWZ)(int)>
struct TrLane {
  int row_off;  // (4g + e) * HD + 4 * (j & 1)
  int t0, t8;   // chunk XOR constants for row bases = 0 and = 8 (mod 16)
  __device__ __forceinline__ TrLane(int lane) {
    const int g = lane >> 5;
    const int e = (lane & 15) >> 2;
    const int x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    row_off = (4 * g + e) * HD + 4 * (lane & 1);
    t0 = x ^ SWZ(4 * g + e);
    t8 = x ^ SWZ(8 + 4 * g + e);
  }
  // element offset of this lane's 4 x bf16 for rows rb + (4g + e), 32-column block cb
  __device__ __forceinline__ int at(int rb, int cb) const {
    return rb * HD + row_off + ((4 * cb) ^ ((rb & 8) ? t8 : t0)) * 8;
  }
};

template <int HD>
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, const TrLane<HD, swz_both<HD>>& tl, int rb, int cb) {
  return __builtin_shufflevector(lds_read_tr(tile + tl.at(rb, cb)), lds_read_tr(tile + tl.at(rb + 8, cb)), 0, 1, 2,
                                 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------------------------ dK dV ----

constexpr int DKDV_STAGES = 3;  // query tiles resident in LDS: one read, one in flight, one draining

template <int HD>
struct DkdvSmem {
  bf16 q[DKDV_STAGES][BWD_BQ * HD];
  bf16 dO[DKDV_STAGES][BWD_BQ * HD];
  float lse[DKDV_STAGES][BWD_BQ];
  float dd[DKDV_STAGES][BWD_BQ];
};

// Work is cut into 32-query blocks u (block u = query rows 32u .. 32u + 31, half u % 2 of query
// tile u / 2), each in three parts:
//   A(u): S and dP accumulators for the wave's 32 keys (16 MFMAs on row operands of the tile),
//   V(u): P = 2^(S c - LSE log2 e) and dS = P (dP - D), rounded to bf16 (vector ALUs),
//   B(u): dV += P^T dO and dK += dS^T Q (16 MFMAs on transposed operands of the tile).
// A step issues A(u+1), V(u) and B(u-1): three independent chains that the wave interleaves. (On
// gfx950 a vector instruction overlaps a running MFMA only when both come from the same wave, so
// the exponentials of one block must sit between the MFMAs of its neighbours.) Query tiles rotate
// through three LDS stages: tile t is read from step 2t-1 (by A) to step 2t+2 (by B), and tile t+2
// is loaded into the stage of tile t-1 right after the barrier between tile t's two steps.
// Causal workgroups run their first two query tiles (the ones crossing the diagonal of some wave)
// block by block with the mask, and the pipeline from the third tile on, where no key of the
// workgroup follows any query.
// One work item of the key-major kernel: the key tile(s) of `item` (ordering below), with the
// workgroup's LDS stages `sm`.
// Rows: dense [B, H, N, d] queries and [B, H_kv, N, d] keys with N rows per sequence, LSE2 and D
// [B, H, N]; or, with VARLEN, packed token rows [T, H, d] and [T, H_kv, d] with sequence b at rows
// cu_seqlens[b] .. cu_seqlens[b+1] - 1 (N the longest length the grid covers), LSE2 and D [H, T].
// Offsets read from cu_seqlens are clamped into [0, T] and lengths to N, as in the forward.
// PREFETCH: the pipelined loop reads each half-step's MFMA operands ahead of its vector work
// (the standalone kernels at d = 128); the fused forward+backward kernel, whose register budget is
// set by its other phases, keeps the compiler's order.
// PLAIN: every tile runs block by block (A, V, B of one block, then the next) instead of through
// the three-part pipeline: the standalone non-causal kernels at d = 64, whose second wave per SIMD
// interleaves with the first in place of the pipeline (the pipelined loop spills 19 registers at
// two waves there). Measured at d = 64, two waves per SIMD against one: [2,16,4096,64] dK/dV
// non-causal 0.379 -> 0.290 ms (plain loop), causal 0.206 -> 0.178 ms (pipeline kept; the plain loop
// gave 0.220), [2,32,2048,64] causal 0.136 -> 0.112, [4,16,1024,64] causal 0.053 -> 0.038.
template <int HD, bool CAUSAL, bool VARLEN = false, bool PREFETCH = (HD == 128),
          bool PLAIN = (HD == 64 && !CAUSAL)>
__device__ __forceinline__ void bwd_dkdv_job(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dg,
    float* __restrict__ dK, float* __restrict__ dV, int H, int group, int N, int n_ktiles, float scale,
    float scale_log2, DkdvSmem<HD>& sm, int item, const int32_t* __restrict__ cu_seqlens = nullptr,
    int T = 0) {
  constexpr int KSTEPS = HD / 16;
  constexpr int CBLK = HD / 32;

  constexpr bool PAIR = CAUSAL && RA_DKDV_PAIR;
  static_assert(!(VARLEN && PAIR), "a ragged batch runs one key tile per workgroup");
  const int per = PAIR ? (n_ktiles + 1) / 2 : n_ktiles;  // workgroups per (sequence, KV head)
  const int pair = item % per;
  const int bhk = item / per;  // (sequence, KV head)
  const int Hkv = H / group;
  const int b = bhk / Hkv;
  const int hk = bhk % Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  int Nb = N, start = 0;  // this sequence's rows and (packed) first row
  if constexpr (VARLEN) {
    start = min(max(cu_seqlens[b], 0), T);
    const int end = min(max(cu_seqlens[b + 1], start), T);
    Nb = min(end - start, N);
  }
  const int rs_q = VARLEN ? H * HD : HD;     // element distance between query rows
  const int rs_kv = VARLEN ? Hkv * HD : HD;  // ... and between key rows

  // With RA_DKDV_PAIR a causal workgroup takes the key tiles (p, n - 1 - p) one after the other so
  // every workgroup carries the same work (as the forward and dQ do). For this kernel, at one
  // workgroup per CU, it measured slower at N >= 4096 (4096: 454 vs 417 us, 8192: 853 vs 735 us)
  // and faster only at 1024, so the default keeps one key tile per workgroup, heaviest first.
  for (int rep = 0; rep < (PAIR ? 2 : 1); ++rep) {
    const int kt = PAIR && rep == 1 ? n_ktiles - 1 - pair : pair;
    if (rep == 1 && kt == pair) break;  // odd tile count: the middle tile runs once
    // every wave is done with the first tile's LDS stages
    if (rep == 1) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (VARLEN && kt * 128 >= Nb) return;  // key tile past this sequence (uniform over the workgroup)
    // K, V, dK, dV rows of this KV head
    const size_t head = VARLEN ? ((size_t)start * Hkv + hk) * HD : (size_t)bhk * N * HD;
    const int kw0 = kt * 128 + w * 32;  // this wave's first key
    const int key = kw0 + l32;          // the key column this lane holds in S and dP

    bf16x8 kf[KSTEPS], vf[KSTEPS];
    if (key < Nb) {
      const bf16x8* ks = reinterpret_cast<const bf16x8*>(K + head + (size_t)key * rs_kv);
      const bf16x8* vs = reinterpret_cast<const bf16x8*>(V + head + (size_t)key * rs_kv);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        kf[kk] = ks[2 * kk + g];
        vf[kk] = vs[2 * kk + g];
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) kf[kk] = vf[kk] = bf16x8{};
    }

    f32x16 dk[CBLK], dv[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) dk[cb] = dv[cb] = f32x16{};

    const TrLane<HD, swz_both<HD>> tl(lane);
    // Row-operand reads (A = Q or dO rows of a 32-query block): row qb*32 + l32, chunk 2kk + g.
    const int row_t = g ^ swz_both<HD>(l32);  // swz_both repeats every 16 rows
    const int row_off = l32 * HD;
    // Query-side rows of the query head currently streamed (set per head of the group below).
    const bf16* Qh = nullptr;
    const bf16* dOh = nullptr;
    const float* LSEh = nullptr;
    const float* Dh = nullptr;
    const int n_qt = (Nb + BWD_BQ - 1) / BWD_BQ;

    auto stage_of = [](int t) { return (t + DKDV_STAGES) % DKDV_STAGES; };  // t >= -1
    auto stage = [&](int qt) {
      const int s = stage_of(qt);
      const int r0 = qt * BWD_BQ;
      if constexpr (VARLEN) {
        const int nv = min(Nb - r0, BWD_BQ);
        stage_rows<HD, BWD_BQ, 4, swz_both<HD>>(Qh + (size_t)r0 * rs_q, rs_q, nv, sm.q[s], w, lane);
        stage_rows<HD, BWD_BQ, 4, swz_both<HD>>(dOh + (size_t)r0 * rs_q, rs_q, nv, sm.dO[s], w, lane);
        if (w == 0) load_to_lds<4>(dma_rsrc(LSEh + r0, nv * 4), lane * 4, sm.lse[s]);
        if (w == 1) load_to_lds<4>(dma_rsrc(Dh + r0, nv * 4), lane * 4, sm.dd[s]);
      } else {
        stage_tile<HD, BWD_BQ, 4, swz_both<HD>>(Qh, r0, N, sm.q[s], w, lane);
        stage_tile<HD, BWD_BQ, 4, swz_both<HD>>(dOh, r0, N, sm.dO[s], w, lane);
        if (w == 0) load_to_lds<4>(dma_rsrc(LSEh + r0, (N - r0) * 4), lane * 4, sm.lse[s]);
        if (w == 1) load_to_lds<4>(dma_rsrc(Dh + r0, (N - r0) * 4), lane * 4, sm.dd[s]);
      }
    };
    // Barrier between the two steps of tile t: this wave's loads of tile t+1 have landed and every
    // wave's reads of tile t-1 have returned; then tile t+2 goes into tile t-1's stage.
    auto mid = [&](int t) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (t + 2 < n_qt) stage(t + 2);
    };

    // Operands of A(u), read from LDS ahead of their MFMAs (the wave holds no other work to cover
    // LDS latency: one wave per SIMD).
    struct AOps {
      bf16x8 q[KSTEPS], d[KSTEPS];
      f32x16 dn;
    };
    // -D of the block's 32 query rows in the dP accumulator layout (rows 32u + 8(r/4) + 4g + r%4): the
    // dP accumulators start there, so they end at dP - D and dS = P (dP - D) is one multiply.
    auto load_dn = [&](int u) {
      const float* dd = &sm.dd[stage_of(u >> 1)][(u & 1) * 32 + 4 * g];
      f32x16 dn;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dd + 8 * rg);
#pragma unroll
        for (int e = 0; e < 4; ++e) dn[4 * rg + e] = d4[e];
      }
      return dn;
    };
    auto load_A = [&](int u, AOps& op) {
      const int s = stage_of(u >> 1);
      op.dn = load_dn(u);
      const bf16* qrow = sm.q[s] + (u & 1) * 32 * HD + row_off;
      const bf16* drow = sm.dO[s] + (u & 1) * 32 * HD + row_off;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int off = ((2 * kk) ^ row_t) * 8;
        op.q[kk] = *reinterpret_cast<const bf16x8*>(qrow + off);
        op.d[kk] = *reinterpret_cast<const bf16x8*>(drow + off);
      }
    };
    auto mfma_A = [&](const AOps& op, f32x16& sacc, f32x16& dpacc) {
      sacc = mfma32(op.q[0], kf[0], f32x16{});
      dpacc = mfma32(op.d[0], vf[0], op.dn);
#pragma unroll
      for (int kk = 1; kk < KSTEPS; ++kk) {
        sacc = mfma32(op.q[kk], kf[kk], sacc);
        dpacc = mfma32(op.d[kk], vf[kk], dpacc);
      }
    };
    auto blk_A = [&](int u, f32x16& sacc, f32x16& dpacc) {
      const int s = stage_of(u >> 1);
      const bf16* qrow = sm.q[s] + (u & 1) * 32 * HD + row_off;
      const bf16* drow = sm.dO[s] + (u & 1) * 32 * HD + row_off;
      sacc = f32x16{};
      dpacc = load_dn(u);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int off = ((2 * kk) ^ row_t) * 8;
        sacc = mfma32(*reinterpret_cast<const bf16x8*>(qrow + off), kf[kk], sacc);
        dpacc = mfma32(*reinterpret_cast<const bf16x8*>(drow + off), vf[kk], dpacc);
      }
    };
    // S, dP lanes: column = key, rows = queries 32u + 8(r/4) + 4g + r%4. P^T and dS^T leave in the
    // A-operand layout of B (lane row = key, k-step hh covers queries 16hh + {4g..4g+3, 8+4g..}).
    auto blk_V = [&](int u, const f32x16& sacc, const f32x16& dpacc, bf16x8 (&pb)[2], bf16x8 (&dsb)[2],
                     bool mask) {
      const int s = stage_of(u >> 1);
      const int qb = u & 1;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sm.lse[s][qb * 32 + 8 * rg + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          float p = fast_exp2(fmaf(sacc[r], scale_log2, -l4[e]));  // l4: LSE * log2 e
          if (mask && key > 32 * u + 8 * rg + 4 * g + e) p = 0.f;
          pb[r >> 3][r & 7] = to_bf16(p);
          dsb[r >> 3][r & 7] = to_bf16(p * dpacc[r]);  // dpacc = dP - D (started at -D)
        }
      }
    };
    // B operands: dO / Q columns 32cb + l32 by transposed read. The first k-step's operands (hh = 0)
    // can be read ahead (load_B0), the second's are read beside the first's MFMAs.
    struct BOps {
      bf16x8 o[CBLK], q[CBLK];
    };
    auto load_B0 = [&](int u, BOps& op) {
      const int s = stage_of(u >> 1);
      const int r0 = (u & 1) * 32;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        op.o[cb] = tr_operand<HD>(sm.dO[s], tl, r0, cb);
        op.q[cb] = tr_operand<HD>(sm.q[s], tl, r0, cb);
      }
    };
    auto mfma_B = [&](int u, const BOps& op, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2]) {
      const int s = stage_of(u >> 1);
      const int r0 = (u & 1) * 32;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        dv[cb] = mfma32(pb[0], op.o[cb], dv[cb]);
        dk[cb] = mfma32(dsb[0], op.q[cb], dk[cb]);
      }
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        dv[cb] = mfma32(pb[1], tr_operand<HD>(sm.dO[s], tl, r0 + 16, cb), dv[cb]);
        dk[cb] = mfma32(dsb[1], tr_operand<HD>(sm.q[s], tl, r0 + 16, cb), dk[cb]);
      }
    };
    auto blk_B = [&](int u, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2]) {
      const int s = stage_of(u >> 1);
      const int r0 = (u & 1) * 32;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) {
          dv[cb] = mfma32(pb[hh], tr_operand<HD>(sm.dO[s], tl, r0 + 16 * hh, cb), dv[cb]);
          dk[cb] = mfma32(dsb[hh], tr_operand<HD>(sm.q[s], tl, r0 + 16 * hh, cb), dk[cb]);
        }
      }
    };

    // The group's query heads run one after another over the same K/V rows; dK and dV accumulate
    // across them in registers, so each element is still written once.
    for (int j = 0; j < group; ++j) {
      if constexpr (VARLEN) {
        const size_t h = (size_t)hk * group + j;
        Qh = Q + ((size_t)start * H + h) * HD;
        dOh = dO + ((size_t)start * H + h) * HD;
        LSEh = LSE2 + h * T + start;
        Dh = Dg + h * T + start;
      } else {
        const size_t qrows = (size_t)b * H + (size_t)hk * group + j;
        Qh = Q + qrows * N * HD;
        dOh = dO + qrows * N * HD;
        LSEh = LSE2 + qrows * N;  // LSE * log2 e, written by the dQ kernel (or the fused forward)
        Dh = Dg + qrows * N;
      }
      // Every wave has finished reading the previous head's tiles before this head's prologue
      // writes LDS.
      if (j > 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int t_first = CAUSAL ? (kt * 128) / BWD_BQ : 0;
      if (!CAUSAL && !PLAIN) {
        // The pipeline's first step applies B to block -1 with zero P and dS; its stage must hold
        // finite values (0 * NaN would poison the accumulators).
        const int s = stage_of(-1);
        bf16x8* zq = reinterpret_cast<bf16x8*>(sm.q[s]);
        bf16x8* zd = reinterpret_cast<bf16x8*>(sm.dO[s]);
        for (int i = tid; i < BWD_BQ * HD / 8; i += BWD_THREADS) zq[i] = zd[i] = bf16x8{};
      }
      stage(t_first);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (t_first + 1 < n_qt) stage(t_first + 1);

      int t = t_first;
      if constexpr (PLAIN) {
        for (; t < n_qt; ++t) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (h == 1) mid(t);
            f32x16 sacc, dpacc;
            bf16x8 pb[2], dsb[2];
            blk_A(2 * t + h, sacc, dpacc);
            blk_V(2 * t + h, sacc, dpacc, pb, dsb, false);
            blk_B(2 * t + h, pb, dsb);
          }
        }
      }
      if (CAUSAL) {
        for (; t < min(n_qt, t_first + 2); ++t) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (h == 1) mid(t);
            f32x16 sacc, dpacc;
            bf16x8 pb[2], dsb[2];
            blk_A(2 * t + h, sacc, dpacc);
            blk_V(2 * t + h, sacc, dpacc, pb, dsb, true);
            blk_B(2 * t + h, pb, dsb);
          }
        }
      }
      if (!PLAIN && t < n_qt) {
        f32x16 sa, da, sb, db;
        bf16x8 pc[2], dc[2], pp[2], dpp[2];
        pp[0] = pp[1] = dpp[0] = dpp[1] = bf16x8{};
        blk_A(2 * t, sa, da);
        for (; t < n_qt; ++t) {
          if constexpr (PREFETCH) {
            // Each half-step reads the operands of its two MFMA groups first (A whole, B's first
            // k-step), so the exponentials and dS of the middle block run while those reads are in
            // flight; the empty asm with a memory clobber keeps the compiler from sinking the reads
            // back next to their MFMAs, where each would wait out its own LDS latency (one wave per
            // SIMD leaves nothing else to cover it). Measured at d = 128: non-causal 0.674 ->
            // 0.590 ms, causal unchanged ([2,16,4096,128]); at d = 64 it was 6% slower, so d = 64
            // keeps the compiler's order below.
            AOps ao;
            BOps bo;
            load_A(2 * t + 1, ao);
            load_B0(2 * t - 1, bo);
            asm volatile("" ::: "memory");
            blk_V(2 * t, sa, da, pc, dc, false);
            mfma_B(2 * t - 1, bo, pp, dpp);
            mfma_A(ao, sb, db);
            mid(t);
            load_A(2 * t + 2, ao);  // past the last tile this reads a drained stage; the result is unused
            load_B0(2 * t, bo);
            asm volatile("" ::: "memory");
            blk_V(2 * t + 1, sb, db, pp, dpp, false);
            mfma_B(2 * t, bo, pc, dc);
            mfma_A(ao, sa, da);
          } else {
            blk_A(2 * t + 1, sb, db);
            blk_V(2 * t, sa, da, pc, dc, false);
            blk_B(2 * t - 1, pp, dpp);
            mid(t);
            blk_A(2 * t + 2, sa, da);  // past the last tile this reads a drained stage; the result is unused
            blk_V(2 * t + 1, sb, db, pp, dpp, false);
            blk_B(2 * t, pc, dc);
          }
        }
        blk_B(2 * n_qt - 1, pp, dpp);
      }
    }

    // dK/dV accumulators: lane column c = 32cb + l32, rows = keys kw0 + 8(r/4) + 4g + r%4.
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = kw0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (kr < Nb) {
          dK[head + (size_t)kr * rs_kv + 32 * cb + l32] = dk[cb][r] * scale;
          dV[head + (size_t)kr * rs_kv + 32 * cb + l32] = dv[cb][r];
        }
      }
    }
  }
}

// --------------------------------------------------------------------------------- dQ ----

template <int HD>
struct DqSmem {
  bf16 k[2][BWD_BK * HD];
  bf16 v[2][BWD_BK * HD];
};

// One work item of the query-major kernel: the query tile(s) of `item` (a pair under a causal
// mask), with the workgroup's LDS stages `sm`.
// ROW_TERMS: the job also computes its rows' D_i = sum_c dO[i,c] O[i,c] from O (bf16) and dO, and
// writes D and LSE * log2 e (what the key-major job streams) to Dg and L2; otherwise it reads D
// from Dg. Row layouts (dense or, with VARLEN, packed by cu_seqlens) are those of the key-major job;
// LSE, Dg and L2 are [B, H, N] or [H, T].
template <int HD, bool CAUSAL, bool ROW_TERMS = false, bool VARLEN = false>
__device__ __forceinline__ void bwd_dq_job(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, float* __restrict__ Dg,
    float* __restrict__ dQ, int H, int group, int N, int n_qtiles, float scale, float scale_log2,
    DqSmem<HD>& sm, int item, const bf16* __restrict__ O = nullptr, float* __restrict__ L2 = nullptr,
    const int32_t* __restrict__ cu_seqlens = nullptr, int T = 0) {
  constexpr int KSTEPS = HD / 16;
  constexpr int CBLK = HD / 32;

  const int per = CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles;  // workgroups per (sequence, head)
  const int pair = item % per;
  const int bh = item / per;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  int Nb = N, start = 0;  // this sequence's rows and (packed) first row
  if constexpr (VARLEN) {
    const int b = bh / H;
    start = min(max(cu_seqlens[b], 0), T);
    const int end = min(max(cu_seqlens[b + 1], start), T);
    Nb = min(end - start, N);
  }
  const int rs_q = VARLEN ? H * HD : HD;                // element distance between query rows
  const int rs_kv = VARLEN ? (H / group) * HD : HD;     // ... and between key rows
  // A ragged batch pairs the tiles of the sequence's own tile count (the grid covers the longest).
  const int nq = VARLEN ? (Nb + 127) / 128 : n_qtiles;
  if (VARLEN && pair >= (CAUSAL ? (nq + 1) / 2 : nq)) return;  // no tile of this sequence left

  // Causal work per query tile grows with its index: a causal workgroup takes the query tiles
  // (n - 1 - p, p) one after the other and every workgroup carries the same work.
  for (int rep = 0; rep < (CAUSAL ? 2 : 1); ++rep) {
    const int qt = CAUSAL && rep == 0 ? nq - 1 - pair : pair;
    if (rep == 1 && qt == nq - 1 - pair) break;  // odd tile count: the middle tile runs once
    // every wave is done with the first tile's LDS stages
    if (rep == 1) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // Q, dO, dQ rows of this query head; its LSE/D rows; the K, V rows of its KV head
    const size_t head = VARLEN ? ((size_t)start * H + bh % H) * HD : (size_t)bh * N * HD;
    const size_t rowbase = VARLEN ? (size_t)(bh % H) * T + start : (size_t)bh * N;
    const size_t kv_head = VARLEN ? ((size_t)start * (H / group) + (bh % H) / group) * HD
                                  : ((size_t)(bh / H) * (H / group) + (bh % H) / group) * N * HD;
    const int q0 = qt * 128 + w * 32;
    const int qi = q0 + l32;

    bf16x8 qf[KSTEPS], df[KSTEPS];
    float lse2 = 0.f, Dq = 0.f;  // rows past N: Q = dO = 0 gives dS = 0
    if (qi < Nb) {
      const bf16x8* qs = reinterpret_cast<const bf16x8*>(Q + head + (size_t)qi * rs_q);
      const bf16x8* ds = reinterpret_cast<const bf16x8*>(dO + head + (size_t)qi * rs_q);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        qf[kk] = qs[2 * kk + g];
        df[kk] = ds[2 * kk + g];
      }
      lse2 = LSE[rowbase + qi] * kLog2e;
      if constexpr (ROW_TERMS) {
        // This lane's half of the row (chunks 2kk + g, as qf and df).
        const bf16x8* os = reinterpret_cast<const bf16x8*>(O + head + (size_t)qi * rs_q);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const bf16x8 a = os[2 * kk + g];
#pragma unroll
          for (int e = 0; e < 8; ++e) Dq = fmaf(to_f32(a[e]), to_f32(df[kk][e]), Dq);
        }
      } else {
        Dq = -Dg[rowbase + qi];  // the workspace holds -D_i
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = df[kk] = bf16x8{};
    }
    if constexpr (ROW_TERMS) {
      Dq += __shfl_xor(Dq, 32, 64);  // the other half of the row (lane l32 + 32)
      if (qi < Nb && g == 0) {
        Dg[rowbase + qi] = -Dq;  // stored negated: the key-major job starts its dP accumulators there
        L2[rowbase + qi] = lse2;  // the row's LSE in log2 units, streamed by the key-major job
      }
    }

    f32x16 acc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) acc[cb] = f32x16{};

    const TrLane<HD, swz_both<HD>> tl(lane);
    const int krow_t = g ^ swz_both<HD>(l32);
    const int vrow_t = g ^ swz_rows<HD>(l32);
    const int row_off = l32 * HD;
    const bf16* Kh = K + kv_head;
    const bf16* Vh = V + kv_head;

    auto stage = [&](int t, int s) {
      if constexpr (VARLEN) {
        const size_t off = (size_t)t * BWD_BK * rs_kv;
        stage_rows<HD, BWD_BK, 4, swz_both<HD>>(Kh + off, rs_kv, Nb - t * BWD_BK, sm.k[s], w, lane);
        stage_rows<HD, BWD_BK, 4, swz_rows<HD>>(Vh + off, rs_kv, Nb - t * BWD_BK, sm.v[s], w, lane);
      } else {
        stage_tile<HD, BWD_BK, 4, swz_both<HD>>(Kh, t * BWD_BK, N, sm.k[s], w, lane);
        stage_tile<HD, BWD_BK, 4, swz_rows<HD>>(Vh, t * BWD_BK, N, sm.v[s], w, lane);
      }
    };

    const int q_end = min(Nb, qt * 128 + 128);
    const int n_kt = CAUSAL ? (q_end + BWD_BK - 1) / BWD_BK : (Nb + BWD_BK - 1) / BWD_BK;
    // One key tile from LDS stage s; MASK applies the causal mask, needed only on the last two key
    // tiles: every key of a tile below them precedes the workgroup's first query (n_kt - 2 <= 2 qt).
    auto tile = [&](int s, int t, auto MASK_) {
      constexpr bool MASK = decltype(MASK_)::value;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 1 < n_kt) stage(t + 1, 1 - s);
      const int k0 = t * BWD_BK;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T and dP^T: lane column = query, rows = keys k0 + 32kb + 8(r/4) + 4g + r%4. The first
        // k-step takes a zero accumulator operand directly (no zero-filled registers).
        // Each MFMA's LDS operand is read two MFMAs ahead; the empty asm statements (memory
        // clobbers) keep the compiler from sinking the reads back next to their MFMAs, where each
        // would wait out its own LDS latency. (Measured with the dQ product's reads below:
        // [2,16,4096,128] causal dQ 0.200 -> 0.193 ms, d = 64 shapes 1.5-6% faster, results bitwise
        // equal.)
        const bf16* krow = sm.k[s] + kb * 32 * HD + row_off;
        const bf16* vrow = sm.v[s] + kb * 32 * HD + row_off;
        constexpr int PF = 2;
        auto rd_row = [&](int i) {  // operand of MFMA i: S^T (i even) or dP^T (i odd), k-step i / 2
          const int kk = i >> 1;
          return (i & 1) ? *reinterpret_cast<const bf16x8*>(vrow + ((2 * kk) ^ vrow_t) * 8)
                         : *reinterpret_cast<const bf16x8*>(krow + ((2 * kk) ^ krow_t) * 8);
        };
        bf16x8 opa[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) opa[i] = rd_row(i);
        asm volatile("" ::: "memory");
        f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
        for (int i = 0; i < 2 * KSTEPS; ++i) {
          const int kk = i >> 1;
          if (i & 1) dpacc = mfma32(opa[i % PF], df[kk], dpacc);
          else sacc = mfma32(opa[i % PF], qf[kk], sacc);
          if (i + PF < 2 * KSTEPS) opa[i % PF] = rd_row(i + PF);
          asm volatile("" ::: "memory");
        }
        // The dQ product's first K^T operands do not depend on dS: read them before the vector work.
        constexpr int PFB = 4;
        auto rd_tr = [&](int i) { return tr_operand<HD>(sm.k[s], tl, 32 * kb + 16 * (i / CBLK), i % CBLK); };
        bf16x8 opb[PFB];
#pragma unroll
        for (int i = 0; i < PFB; ++i) opb[i] = rd_tr(i);
        asm volatile("" ::: "memory");
        bf16x8 dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(sacc[r], scale_log2, -lse2));
          if (MASK && k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3) > qi) p = 0.f;
          dsb[r >> 3][r & 7] = to_bf16(p * (dpacc[r] - Dq));
        }
        // dQ^T += K^T dS^T for this block's 32 keys: A = K^T (rows c = 32cb + l32 by transposed
        // read of the key tile), k-steps 2kb, 2kb + 1; MFMA i takes k-step i / CBLK, block i % CBLK.
#pragma unroll
        for (int i = 0; i < 2 * CBLK; ++i) {
          acc[i % CBLK] = mfma32(opb[i % PFB], dsb[i / CBLK], acc[i % CBLK]);
          if (i + PFB < 2 * CBLK) opb[i % PFB] = rd_tr(i + PFB);
          asm volatile("" ::: "memory");
        }
      }
    };
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    const int t_mask = CAUSAL ? max(0, n_kt - 2) : n_kt;
    stage(0, 0);
    int t = 0;
    // At d = 128 without the mask, two tiles per trip: each tile's LDS stage is then a constant that
    // folds into the LDS reads' immediate offsets, where a stage chosen at run time cost 42 address
    // instructions per tile (the kernel has no registers left to hold the per-lane offsets of both
    // stages). The causal kernel keeps one tile per trip: with the masked tiles' loop beside it the
    // unrolled loop spilled 48 bytes per lane, and the spill-free loop runs as fast. At d = 64 the
    // unrolled loop needs registers beyond three waves per SIMD.
    if constexpr (HD == 128 && !CAUSAL) {
      for (; t + 1 < t_mask; t += 2) {  // t starts at 0: stage 0 first
        tile(0, t, NoMask{});
        tile(1, t + 1, NoMask{});
      }
    }
    for (; t < t_mask; ++t) tile(t & 1, t, NoMask{});
    for (; t < n_kt; ++t) tile(t & 1, t, Mask{});

    if (qi < Nb) {
      float* out = dQ + head + (size_t)qi * rs_q;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          *reinterpret_cast<f32x4*>(out + 32 * cb + 8 * rg + 4 * g) =
              f32x4{acc[cb][4 * rg] * scale, acc[cb][4 * rg + 1] * scale, acc[cb][4 * rg + 2] * scale,
                    acc[cb][4 * rg + 3] * scale};
        }
      }
    }
  }
}

}  // namespace ra
