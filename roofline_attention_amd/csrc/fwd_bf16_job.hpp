// Fused tiled attention forward for bf16 inputs on gfx950 (MFMA 32x32x16 bf16, fp32 accumulate).
//
// Schedule ("Why Fast GPUs Still Wait for Memory", section "FlashAttention is an IO algorithm"):
// a workgroup owns FWD_BR query rows of one (batch, head); it streams every K/V tile of FWD_BC
// keys through LDS, keeps a running row maximum and normaliser, rescales its output accumulator
// when the maximum moves, and never writes S or P to memory. Causal workgroups stop at the
// diagonal and mask only the tiles that straddle it (same page, note on causal masking).
//
// gfx950 mapping:
//   * 4 waves x 32 query rows. Each wave keeps its Q rows in registers as the MFMA B operand.
//   * Scores are produced transposed, S^T = K Q^T (A = K rows from LDS, B = Q), so each lane holds
//     one query row: the row max needs one v_permlane32_swap, and the probabilities leave the
//     accumulator already in the B-operand layout of O^T = V^T P^T.
//   * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ... lds, no VGPR staging;
//     the buffer range check zero-fills rows past the sequence end).
//     Each wave instruction fills 1 KB of LDS in lane order, so bank conflicts are avoided by an
//     XOR swizzle of the 16-byte chunks within a row instead of padding.
//   * The V^T operand of O^T = V^T P^T comes from ds_read_b64_tr_b16, which transposes 16-bit
//     elements across each 16-lane group, so V is never transposed in memory.
//   * Software pipeline: while the softmax of tile j runs on the vector ALUs, the score MFMAs of
//     tile j+1 are issued beside it, so one wave keeps the matrix cores fed (a vector instruction
//     overlaps an MFMA on gfx950 only when both come from the same wave). K is therefore loaded
//     one tile ahead of V (two LDS stages each, one barrier per tile).
//   * The running maximum is only raised when a tile's maximum exceeds it by more than 8 (log2
//     units); the numerator and the normaliser always share the same reference, so the result is
//     unchanged while the output rescale is skipped on almost every tile. The probabilities are
//     first taken against the current reference; only when some lane's bf16 row sum reaches 2^8
//     (so a probability might exceed 2^8, or the reference is still unset) does the tile take the
//     exact path: row maximum, raise decision, rescale, probabilities again. Below 2^8 no raise is
//     possible, so the result is that of deciding on every tile, without the maximum on most.
//   * Masks are applied only on tiles that cross the causal diagonal or the sequence end.
//   * Workgroup ids are remapped so the query tiles of one head run on one XCD (shared L2); a causal
//     workgroup runs a heavy and a light query tile so every workgroup carries the same work.
#pragma once

#include <float.h>
#include <math.h>

#include "common.hpp"
#include "lds_tile.hpp"

namespace ra {

#ifndef RA_FWD_WAVES
#define RA_FWD_WAVES 4
#endif
// Waves per workgroup, 32 query rows each. Eight waves (one workgroup per CU sharing each K/V tile)
// measured within 1% of four ([2,32,4096,128]: 482 vs 489 us non-causal, 271 vs 270 us causal,
// where eight spill 13 registers), so four stay.
constexpr int FWD_WAVES = RA_FWD_WAVES;
constexpr int FWD_BR = 32 * FWD_WAVES;
constexpr int FWD_BC = 64;
constexpr int FWD_THREADS = 64 * FWD_WAVES;
constexpr float kLazyRescale = 8.0f;  // log2 units: P values stay below 2^8

// LDS tiles: [2 stages][FWD_BC rows][HD] bf16, unpadded. The 16-byte chunk c of row r is stored
// at chunk position c ^ swz(r): swz_k spreads the 32 rows one MFMA A-operand read touches over
// the banks; swz_v spreads the 4-row footprint of a transposed read (32 lanes per LDS cycle).
template <int HD>
struct FwdSmem {
  bf16 k[2][FWD_BC * HD];
  bf16 v[2][FWD_BC * HD];
};

template <int HD>
__device__ __forceinline__ int swz_k(int r) {
  // A 16-lane b128 read touches rows r..r+15 at one chunk. 256-byte rows (d = 128) all start in
  // bank 0, so 16 distinct chunk positions suffice; 128-byte rows (d = 64) alternate between the
  // two bank halves by row parity, so rows r and r+8 need distinct positions: key the swizzle on
  // r / 2 (period 16 rows either way).
  if constexpr (HD == 128) return r & 15;
  else return (r >> 1) & 7;
}
template <int HD>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (HD == 128) return 4 * (r & 3) + 2 * ((r >> 1) & 1);
  else return (2 * r) & 7;
}

// max over the lane pair (l, l ^ 32) that shares one query row
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// sum over the same lane pair (one VALU exchange; no lane-index address as for a shuffle)
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// One work item of the forward: query tile `item` of the grid's ordering (a pair of tiles under a
// causal mask). The standalone kernel's item (FUSED false) declares its LDS tiles here; inside the
// fused forward+backward kernel (FUSED true) the tiles live in the caller's LDS `ext`, and the
// epilogue also writes, per query row, the backward's inputs D_i = sum_c dO[i,c] O[i,c] (O as
// stored, bf16) and LSE_i * log2 e, so no separate pass over O and dO is needed. (Naming the
// standalone tiles as a __shared__ variable of this function keeps the kernel's register
// allocation as it was with the tiles declared in the kernel; reaching them through a pointer or a
// reference parameter cost the ragged causal kernel two spilled registers.)
template <int HD, bool CAUSAL, bool VARLEN, bool FUSED>
__device__ __forceinline__ void fwd_bf16_job(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                             const bf16* __restrict__ V, bf16* __restrict__ O,
                                             float* __restrict__ LSE, const int32_t* __restrict__ cu_seqlens,
                                             int T, int H, int group, int N, int n_qtiles, float scale_log2,
                                             FwdSmem<HD>* ext, int item, const bf16* __restrict__ dO,
                                             float* __restrict__ Dg, float* __restrict__ L2,
                                             int only_rep = -1) {
  __shared__ FwdSmem<HD> own;  // unreferenced, hence not allocated, when FUSED
  FwdSmem<HD>& sm = FUSED ? *ext : own;
  constexpr int KSTEPS = HD / 16;  // MFMA k-steps over the head dimension
  constexpr int CBLK = HD / 32;    // 32-wide head-dimension blocks of O^T
  constexpr int CHUNKS = HD / 8;   // 16-byte chunks per row
  constexpr int RPI = 1024 / (HD * 2);   // rows per direct-load wave instruction
  constexpr int BLOCKS = FWD_BC / RPI;   // wave instructions per tensor per tile

  const int per_head = CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles;  // workgroups per (sequence, head)
  const int pair = item % per_head;
  const int bh = item / per_head;
  const int h = bh % H;
  const int b = bh / H;
  const int Hkv = H / group;
  const int hk = h / group;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  // Rows of this (sequence, head): dense [B,H,N,d] / [B,H_kv,N,d] with N rows per sequence, or
  // packed [T,H,d] / [T,H_kv,d] with sequence b at rows cu_seqlens[b] .. cu_seqlens[b+1] - 1 (N is
  // then the longest length the grid covers). Offsets read from the device array are clamped into
  // [0, T] and lengths to N, so no access leaves the tensors whatever they hold. Row strides and
  // bases are in elements; LSE is [B,H,N] or [H,T].
  int Nb = N;
  size_t q_base, kv_base, lse_base;
  int rs_q = HD, rs_kv = HD;
  if constexpr (VARLEN) {
    const int start = min(max(cu_seqlens[b], 0), T);
    const int end = min(max(cu_seqlens[b + 1], start), T);
    Nb = min(end - start, N);
    q_base = ((size_t)start * H + h) * HD;
    kv_base = ((size_t)start * Hkv + hk) * HD;
    lse_base = (size_t)h * T + start;
    rs_q = H * HD;
    rs_kv = Hkv * HD;
  } else {
    q_base = ((size_t)b * H + h) * (size_t)N * HD;
    kv_base = ((size_t)b * Hkv + hk) * (size_t)N * HD;
    lse_base = ((size_t)b * H + h) * N;
  }
  // Causal work per query tile grows with its index, so a causal workgroup takes the pair of tiles
  // (n - 1 - p, p): every workgroup then does the same work and the last round has no long tail
  // (measured: 75% of workgroup slots busy with one tile per workgroup, heaviest first). n counts
  // the tiles of this workgroup's own sequence: in a ragged batch the grid covers the longest one,
  // and pairing a shorter sequence against that count would give a few workgroups all its heavy
  // tiles (measured: twice the time of the ragged workload).
  // only_rep 0 or 1 runs just the heavy or just the light tile of the pair (a small grid then
  // launches each pair as two workgroups, filling twice the workgroup slots); -1 runs both.
  const int n_own = VARLEN ? (Nb + FWD_BR - 1) / FWD_BR : n_qtiles;
  if (CAUSAL && pair >= (n_own + 1) / 2) return;  // no tile of this sequence left for this pair slot
  for (int rep = (only_rep == 1 ? 1 : 0); rep < (CAUSAL && only_rep != 0 ? 2 : 1); ++rep) {
    const int qt = CAUSAL && rep == 0 ? n_own - 1 - pair : pair;
    if (rep == 1 && qt == n_own - 1 - pair) break;  // odd tile count: the middle tile runs once
    if (qt * FWD_BR >= Nb) continue;  // query tile past this sequence (uniform over the workgroup)
    if (rep == 1 && only_rep < 0) __syncthreads();  // every wave is done with the first tile's LDS stages
    const int q0 = qt * FWD_BR + w * 32;
    const int qi = q0 + l32;

    // The sign of the scale is folded into Q (exact) and its magnitude is kept >= FLT_MIN, so the
    // exponent factor c is positive: the maximum of the raw scores gives the maximum of the scaled
    // ones, and masked raw scores of -inf scale to -inf (a zero scale then yields exp2(0) = 1 for
    // every kept key, the uniform average).
    const bool neg = scale_log2 < 0.f;
    const float c = fmaxf(neg ? -scale_log2 : scale_log2, FLT_MIN);
    bf16x8 qf[KSTEPS];
    if (qi < Nb) {
      // row address from the lane index, as in the epilogue: a causal workgroup's second tile then
      // needs no pointer kept from the first
      const int lane_q = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
      const bf16x8* src = reinterpret_cast<const bf16x8*>(Q + q_base + (size_t)(q0 + (lane_q & 31)) * rs_q);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = src[2 * kk + (lane_q >> 5)];
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = bf16x8{};
    }
    // The sign flip: one XOR of the packed sign bits per dword, under a wave-uniform branch outside
    // the divergent row test (an element-wise negation inside it cost four instructions per pair,
    // issued whatever the sign).
    if (neg) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[kk]) ^ 0x80008000u);
    }

    const int q_end = min(Nb, qt * FWD_BR + FWD_BR);
    const int n_kt = CAUSAL ? (q_end + FWD_BC - 1) / FWD_BC : (Nb + FWD_BC - 1) / FWD_BC;

    // Direct-to-LDS staging: wave w issues blocks w, w + 4, ... of a tile (RPI rows each). Lane i
    // fills row blk*RPI + i / CHUNKS at chunk position i % CHUNKS with global chunk
    // position ^ swz(row). The swizzles repeat within FWD_WAVES*RPI rows, so a lane's offset moves by
    // BLK_BYTES from one of its blocks to the next. The buffer resource of tile kt starts at its
    // first row and ends with the last byte of the tile's last row inside the sequence, so rows past
    // the sequence end load as zeros.
    const int BLK_BYTES = FWD_WAVES * RPI * rs_kv * 2;  // byte distance between this wave's blocks
    const int st_row = w * RPI + lane / CHUNKS;
    const int k_voff = (st_row * rs_kv + (((lane % CHUNKS) ^ swz_k<HD>(st_row)) * 8)) * 2;
    const int v_voff = (st_row * rs_kv + (((lane % CHUNKS) ^ swz_v<HD>(st_row)) * 8)) * 2;
    const bf16* k_head = K + kv_base;
    const bf16* v_head = V + kv_base;
    auto tile_bytes = [&](int row0) { return (min(Nb - row0, FWD_BC) - 1) * rs_kv * 2 + HD * 2; };
    auto issue_k = [&](int kt, int stage) {
      const int row0 = kt * FWD_BC;
      const u32x4 rsrc = dma_rsrc(k_head + (size_t)row0 * rs_kv, tile_bytes(row0));
#pragma unroll
      for (int u = 0; u < BLOCKS / FWD_WAVES; ++u) {
        if (u == 0) load_to_lds<16>(rsrc, k_voff, &sm.k[stage][w * RPI * HD]);
        else load_to_lds16_so(rsrc, k_voff, u * BLK_BYTES, &sm.k[stage][(u * FWD_WAVES + w) * RPI * HD]);
      }
    };
    auto issue_v = [&](int kt, int stage) {
      const int row0 = kt * FWD_BC;
      const u32x4 rsrc = dma_rsrc(v_head + (size_t)row0 * rs_kv, tile_bytes(row0));
#pragma unroll
      for (int u = 0; u < BLOCKS / FWD_WAVES; ++u) {
        if (u == 0) load_to_lds<16>(rsrc, v_voff, &sm.v[stage][w * RPI * HD]);
        else load_to_lds16_so(rsrc, v_voff, u * BLK_BYTES, &sm.v[stage][(u * FWD_WAVES + w) * RPI * HD]);
      }
    };

    // K A-operand read (S^T block kb, k-step kk): row 32kb + l32, chunk 2kk + g at position
    // (2kk + g) ^ swz_k(l32) (32kb is a multiple of the swizzle period).
    const int k_lane = l32 * HD;
    const int k_t = g ^ swz_k<HD>(l32);
    // Transposed V read: in its 16-lane group, source lane 4e + j points at key row (4g + e) of the
    // k-step and element column 16 * ((lane / 16) % 2) + 4j of the 32-column block; the read returns
    // V[4 keys][one column]. Key rows of a k-step start at multiples of 8, so the swizzle of row
    // 4g + e is a lane constant.
    const int v_row = 4 * g + ((lane & 15) >> 2);
    const int v_x = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within the 32-column block
    const int v_t = v_x ^ swz_v<HD>(v_row);
    const int v_lane = v_row * HD + 4 * (lane & 1);

    // S^T for one tile: block kb rows = keys 32kb + 8(r/4) + 4g + r%4, column = this lane's query.
    auto scores = [&](const bf16* kbuf, f32x16 (&s)[2]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
        const bf16* krow = &kbuf[32 * kb * HD + k_lane];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
          s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(krow + ((2 * kk) ^ k_t) * 8), qf[kk], s[kb]);
      }
    };

    // One 32-key half (block kb) of S^T for one tile. At d = 128 each K operand is read two MFMAs
    // ahead, pinned there by empty asm statements with memory clobbers (the compiler otherwise
    // places some reads right before their MFMA, which then waits the LDS latency): about 1%
    // on the 4k shapes, bitwise the same; at d = 64 it measured 0.3-0.6% slower.
    auto scores_half = [&](const bf16* kbuf, f32x16 (&s)[2], int kb) {
      s[kb] = f32x16{};
      const bf16* krow = &kbuf[32 * kb * HD + k_lane];
      if constexpr (HD == 128) {
        constexpr int SPF = 2;
        bf16x8 op[SPF];
#pragma unroll
        for (int i = 0; i < SPF; ++i) op[i] = *reinterpret_cast<const bf16x8*>(krow + ((2 * i) ^ k_t) * 8);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          s[kb] = mfma32(op[kk % SPF], qf[kk], s[kb]);
          if (kk + SPF < KSTEPS) op[kk % SPF] = *reinterpret_cast<const bf16x8*>(krow + ((2 * (kk + SPF)) ^ k_t) * 8);
          asm volatile("" ::: "memory");
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
          s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(krow + ((2 * kk) ^ k_t) * 8), qf[kk], s[kb]);
      }
    };

    f32x16 oacc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
    float m_run = -INFINITY;  // reference maximum (log2 units) shared by numerator and normaliser
    float l_run = 0.f;        // this lane's share of the normaliser

    // Masks raw scores of a boundary tile with -inf (causal diagonal, sequence end). Slot (kb, r) of
    // this lane holds key k0 + 4g + off(kb, r), off a compile-time constant below 64, and a key is
    // kept when it is at most the lane's last visible key (its query row under the causal mask, and
    // never past the sequence end): one compare against a lane threshold and one select per score.
    auto apply_mask = [&](int k0, f32x16 (&s)[2]) {
      const int last_key = CAUSAL ? min(qi, Nb - 1) : Nb - 1;
      const int lim = last_key - k0 - 4 * g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
          if (off > lim) s[kb][r] = -INFINITY;
        }
      }
    };

    // Exact lazy-raise decision for raw scores s: the tile maximum, the new reference maximum and
    // the rescale factor alpha; returns whether any lane of the wave raised its reference (the
    // caller then rescales the output accumulator).
    auto decide = [&](const f32x16 (&s)[2], float& alpha) {
      // Row maximum over the 32 scores as a tree of 3-input maxima. fmaximum (NaN-propagating)
      // equals fmaxf on the finite or -inf scores here and needs no NaN-quieting of its inputs.
      float m1[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int a = 3 * i, b = 3 * i + 1, c3 = 3 * i + 2;
        m1[i] = vmax3(s[a >> 4][a & 15], s[b >> 4][b & 15], s[c3 >> 4][c3 & 15]);
      }
      m1[10] = __builtin_elementwise_maximum(s[1][14], s[1][15]);
      const float m2a = vmax3(m1[0], m1[1], m1[2]), m2b = vmax3(m1[3], m1[4], m1[5]);
      const float m2c = vmax3(m1[6], m1[7], m1[8]), m2d = __builtin_elementwise_maximum(m1[9], m1[10]);
      const float rmax = vmax3(m2a, m2b, __builtin_elementwise_maximum(m2c, m2d));
      // Tile 0 always holds key 0, which every query row keeps, so m_run is finite after it.
      const float tmax = pair_max(rmax) * c;
      const bool raise = tmax > m_run + kLazyRescale;
      const float m_new = raise ? tmax : m_run;
      alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      return __builtin_amdgcn_ballot_w64(raise) != 0;
    };
    // P^T = 2^(s c - m_run) in the B-operand layout (k-step ks = 2kb + hh takes accumulator slots
    // 8hh..8hh+7); returns this lane's sum of the bf16-rounded probabilities, which are what
    // multiplies V (bf16 dot products with (1, 1), fp32 accumulation).
    auto probs = [&](const f32x16 (&s)[2], bf16x8 (&pf)[4]) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pf[2 * kb + (r >> 3)][r & 7] = to_bf16(fast_exp2(fmaf(s[kb][r], c, -m_run)));
      }
      float tsum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) tsum = bf16_pair_sum(pf[i][e], pf[i][e + 1], tsum);
      }
      return tsum;
    };
    // Online-softmax step on raw scores s: P^T of the tile and the normaliser update, the output
    // rescaled when the reference rises. Against the current reference every probability of a
    // lane is at most its row sum, so a sum below 2^8 rules out a raise (any score more than 8 above
    // the reference gives a probability that rounds to at least 2^8); otherwise (or on an infinite
    // or NaN sum: reference unset) the exact decision runs and the probabilities are taken again.
    auto softmax = [&](const f32x16 (&s)[2], bf16x8 (&pf)[4]) {
      float tsum = probs(s, pf);
      if (__builtin_amdgcn_ballot_w64(!(tsum < 256.f)) != 0) {
        float alpha;
        if (decide(s, alpha)) {
#pragma unroll
          for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
        }
        l_run *= alpha;
        tsum = probs(s, pf);
      }
      l_run += tsum;
    };

    // O^T += V^T P^T. A operand: lane row c = 32cb + l32, keys 32kb + 16hh + {4g..4g+3, 8+4g..8+4g+3}.
    // At d = 64 the V^T operands are read four MFMAs ahead (pinned as above): 3% on [4,16,1024,64]
    // causal, bitwise the same; at d = 128 no gain.
    auto pv = [&](const bf16* vbuf, const bf16x8 (&pf)[4]) {
      if constexpr (HD == 64) {
        constexpr int VPF = 4;
        auto rdv = [&](int i) {  // operand of MFMA i: k-step i / CBLK, output block i % CBLK
          const int ks = i / CBLK, cb = i % CBLK;
          const bf16* vp = &vbuf[(32 * (ks >> 1) + 16 * (ks & 1)) * HD + v_lane + ((4 * cb) ^ v_t) * 8];
          return __builtin_shufflevector(lds_read_tr(vp), lds_read_tr(vp + 8 * HD), 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 op[VPF];
#pragma unroll
        for (int i = 0; i < VPF; ++i) op[i] = rdv(i);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 4 * CBLK; ++i) {
          oacc[i % CBLK] = mfma32(op[i % VPF], pf[i / CBLK], oacc[i % CBLK]);
          if (i + VPF < 4 * CBLK) op[i % VPF] = rdv(i + VPF);
          asm volatile("" ::: "memory");
        }
        return;
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks >> 1;
        const int hh = ks & 1;
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) {
          const bf16* vp = &vbuf[(32 * kb + 16 * hh) * HD + v_lane + ((4 * cb) ^ v_t) * 8];
          const bf16x8 va =
              __builtin_shufflevector(lds_read_tr(vp), lds_read_tr(vp + 8 * HD), 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[cb] = mfma32(va, pf[ks], oacc[cb]);
        }
      }
    };

    auto is_boundary = [&](int kt) {
      const int k0 = kt * FWD_BC;
      return (k0 + FWD_BC > Nb) || (CAUSAL && k0 + FWD_BC - 1 > q0);
    };

    // Prologue: K0, V0 and K1 in flight, then S^T of tile 0.
    issue_k(0, 0);
    issue_v(0, 0);
    if (n_kt > 1) issue_k(1, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 s_cur[2];
    scores(sm.k[0], s_cur);
    __syncthreads();  // every wave has read K0 before its stage is reused for K2

    // One pipelined step. Entering it: sc = S^T of tile kt, K_{kt+1} and V_kt in LDS. It issues the
    // loads of V_{kt+1} and K_{kt+2}, the score MFMAs of tile kt+1 (into sn) together with the
    // softmax of tile kt, then O += V_kt P_kt, and ends at a barrier.
    auto step = [&](int kt, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      issue_v(kt + 1, (kt + 1) & 1);
      if (kt + 2 < n_kt) issue_k(kt + 2, kt & 1);
      if (is_boundary(kt)) apply_mask(kt * FWD_BC, sc);
      bf16x8 pf[4];
      // The (rare) exact path of the softmax is a branch, and the compiler interleaves vector work
      // only with MFMAs of the same basic block: the first half of tile kt + 1's score MFMAs goes
      // with the exponentials before the branch, the second half with O += V P of tile kt after it.
      scores_half(sm.k[(kt + 1) & 1], sn, 0);  // matrix cores: tile kt + 1, keys 0..31
      softmax(sc, pf);                          // vector ALUs: tile kt
      scores_half(sm.k[(kt + 1) & 1], sn, 1);  // keys 32..63
      pv(sm.v[kt & 1], pf);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of V_{kt+1}, K_{kt+2} have landed
      __syncthreads();                // ... and every wave's; stages read in this step are free
    };
    // The last tile: softmax and O += V P only.
    auto last = [&](int kt, f32x16 (&sc)[2]) {
      // Under a causal mask the last key tile can lie wholly above this wave's rows (the first
      // waves of a workgroup on its second diagonal tile): every probability is 0, nothing to add.
      if (CAUSAL && kt * FWD_BC > q0 + 31) return;
      if (is_boundary(kt)) apply_mask(kt * FWD_BC, sc);
      bf16x8 pf[4];
      float alpha;  // the exact path directly: one tile, nothing to overlap
      if (decide(sc, alpha)) {
#pragma unroll
        for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
      }
      l_run = fmaf(l_run, alpha, probs(sc, pf));
      pv(sm.v[kt & 1], pf);
    };
    // Two steps per trip so the two score buffers trade roles instead of being copied.
    f32x16 s_alt[2];
    int kt = 0;
    for (; kt + 2 < n_kt; kt += 2) {
      step(kt, s_cur, s_alt);
      step(kt + 1, s_alt, s_cur);
    }
    // One last() on one buffer: inlining it on either buffer made the compiler merge the two copies
    // with register shuffles and spill around the rescale branch.
    if (kt + 1 < n_kt) {
      step(kt, s_cur, s_alt);
      s_cur[0] = s_alt[0];
      s_cur[1] = s_alt[1];
      ++kt;
    }
    last(kt, s_cur);

    l_run = pair_sum(l_run);
    // The epilogue takes its row from the lane index (v_mbcnt) instead of the prologue's
    // registers, so no per-lane address has to stay live across the tile loop for it.
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int qi_e = q0 + (lane_e & 31);
    const int g_e = lane_e >> 5;
    if (qi_e < Nb) {
      const float inv = 1.f / l_run;
      bf16* orow = O + q_base + (size_t)qi_e * rs_q;
      float dsum = 0.f;  // this lane's half of D_i (FUSED)
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          bf16x4 t = {to_bf16(oacc[cb][4 * rg + 0] * inv), to_bf16(oacc[cb][4 * rg + 1] * inv),
                      to_bf16(oacc[cb][4 * rg + 2] * inv), to_bf16(oacc[cb][4 * rg + 3] * inv)};
          *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * rg + 4 * g_e) = t;
          if constexpr (FUSED) {
            const bf16x4 d4 =
                *reinterpret_cast<const bf16x4*>(dO + q_base + (size_t)qi_e * rs_q + 32 * cb + 8 * rg + 4 * g_e);
#pragma unroll
            for (int e = 0; e < 4; ++e) dsum = fmaf(to_f32(t[e]), to_f32(d4[e]), dsum);
          }
        }
      }
      if constexpr (FUSED) {
        const float lse_row = (m_run + log2f(l_run)) * kLn2;
        dsum = pair_sum(dsum);  // lanes l and l ^ 32 hold the two column halves of row qi
        if (g_e == 0) {
          LSE[lse_base + qi_e] = lse_row;
          Dg[lse_base + qi_e] = -dsum;  // the backward's workspace holds -D_i
          L2[lse_base + qi_e] = lse_row * kLog2e;
        }
      } else {
        if (LSE != nullptr && g_e == 0) LSE[lse_base + qi_e] = (m_run + log2f(l_run)) * kLn2;
      }
    }
  }
}

}  // namespace ra
