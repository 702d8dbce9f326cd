// Fused tiled attention forward for fp8 (OCP E4M3) inputs on gfx950, d = 64 or 128.
//
// Same schedule as the bf16 forward ("Why Fast GPUs Still Wait for Memory", section
// "FlashAttention is an IO algorithm"): a workgroup owns 128 query rows of one (batch, head),
// streams K/V tiles of 64 keys through LDS with an online softmax, and never writes S or P to
// memory. What changes is the matrix instruction: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies
// E4M3 operands at twice the bf16 rate (the doubled compute ceiling of fp8, same page, section
// "pi is the top of a stack" and Table 1), 64 products deep per instruction.
//
// gfx950 mapping:
//   * 4 waves x 32 query rows; Q rows stay in registers as the B operand of S^T = K Q^T. Each lane
//     holds 32 code bytes per instruction (d = 64kk + 32g .. +31 for lane half g), K rows are read
//     with the same byte order, so both operands agree on which d each byte slot carries.
//   * The accumulator of S^T leaves each lane with 32 keys of one query row, which is exactly the
//     32-byte B operand of O^T = V^T P^T: the probabilities are rounded to E4M3 in place
//     (v_cvt_pk_fp8_f32, round to nearest even) and one 64-key MFMA per 32 output columns follows.
//   * V^T comes from ds_read_b64_tr_b8: in each 16-lane group, source lane 2k + b supplies key row
//     k of the read and byte column 8b .. 8b+7, and result lane t receives column t of those 8
//     keys. Four such reads give the 32 keys of a lane in the order of its probabilities.
//   * K and V tiles (d-byte rows) go straight from HBM into LDS, 16-byte chunks XOR-swizzled so
//     that the K row reads (16 rows per b128 phase) and the transposed V reads (8 rows x 2 chunks
//     per 32 lanes) hit distinct banks.
//   * P is formed as 2^(s - m + 6), the reference m always some tile's maximum (so at most the
//     row's): every P down to 2^-12 of it is a normal E4M3 number.
//   * The normaliser is the sum of the E4M3-rounded P, the values that multiply V, and it is taken
//     on the matrix core: one more 64-key MFMA per tile, with an all-ones A operand, leaves every
//     lane the column sum of its query. The kernel is bound by its vector work, not by the matrix
//     core, so one MFMA (64 cycles) in place of 31 float32 adds per lane is a net gain.
//   * The probabilities are taken against the current reference first. The E4M3 conversion does not
//     saturate (a value above 464 becomes the NaN code) and the matrix unit carries a NaN byte into
//     its query's column sum, so a NaN sum flags a probability that does not fit; only then (and on
//     a row's first tile) does the tile compute its maximum, raise the reference when the maximum
//     exceeds it by more than 2 (log2 units), rescale O and take the probabilities again. Every P
//     that multiplies V is a finite E4M3 value of at most 448.
//   * Descales: q and k descales fold into the score factor, the v descale into the final 1 / l.
#include <float.h>
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace ra {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int F8_BR = 128;
constexpr int F8_BC = 64;
constexpr int F8_THREADS = 256;
constexpr float kLazy = 2.0f;       // log2 units
constexpr float kPOffset = 6.0f;    // log2 of the factor P carries while on chip

template <int HD>
struct Fp8Smem {  // HD = head dimension = bytes per K/V row
  uint8_t k[2][F8_BC * HD];
  uint8_t v[2][F8_BC * HD];
};

// Chunk swizzles (16-byte chunks; 64 banks x 4 bytes = 16 chunk slots). 128-byte rows alternate
// between the two halves of the banks by parity, 64-byte rows cycle through four quarters.
// K: a b128 phase reads chunk c of 16 consecutive rows, so rows that share a bank slot (one parity
// at d = 128, one residue mod 4 at d = 64) need distinct positions. V: a transposed read touches
// rows {0..3, 8..11} + 4g at two adjacent chunks per 32 lanes; rows sharing a slot then need
// positions that differ above bit 0.
template <int HD>
__device__ __forceinline__ int swz8_k(int r) {
  if constexpr (HD == 128) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}
template <int HD>
__device__ __forceinline__ int swz8_v(int r) {
  if constexpr (HD == 128) return 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1);
  else return 2 * ((r >> 3) & 1);
}

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // operand formats 0 (E4M3) and unit block scales (E8M0 code 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 __attribute__((address_space(3)))*)(p));
}

__device__ __forceinline__ i32x8 cat16(const uint4& a, const uint4& b) {
  return i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__device__ __forceinline__ float pair_max8(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(F8_THREADS, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int H, int group, int N, int n_qtiles, float scale_log2,
    float v_descale, int split_pairs) {
  __shared__ Fp8Smem<HD> sm;
  constexpr int KK = HD / 64;          // 64-deep MFMAs per 32x32 score block
  constexpr int CBLK = HD / 32;        // 32-wide head-dimension blocks of O^T
  constexpr int CHUNKS = HD / 16;      // 16-byte chunks per row
  constexpr int RPI = 1024 / HD;       // rows per direct-load wave instruction (8 or 16)
  constexpr int BLOCKS = F8_BC / RPI;  // wave instructions per tensor per tile (8 or 4)

  // With split_pairs the grid holds each causal pair twice: workgroups L and L + half run its heavy
  // and its light tile (only_rep 0 and 1); otherwise one workgroup runs both (only_rep -1).
  const int half = split_pairs ? (int)gridDim.x / 2 : (int)gridDim.x;
  const int item = xcd_remap(blockIdx.x % half, half);
  const int only_rep = split_pairs ? (int)(blockIdx.x / half) : -1;
  const int per_head = CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles;
  const int pair = item % per_head;
  const int bh = item / per_head;
  const int h = bh % H;
  const int b = bh / H;
  const int Hkv = H / group;
  const int hk = h / group;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const size_t q_base = ((size_t)b * H + h) * (size_t)N * HD;
  const size_t kv_base = ((size_t)b * Hkv + hk) * (size_t)N * HD;
  const size_t lse_base = ((size_t)b * H + h) * N;

  // Causal workgroups take the query tiles (n - 1 - p, p) so every workgroup does the same work.
  for (int rep = (only_rep == 1 ? 1 : 0); rep < (CAUSAL && only_rep != 0 ? 2 : 1); ++rep) {
    const int qt = CAUSAL && rep == 0 ? n_qtiles - 1 - pair : pair;
    if (rep == 1 && qt == n_qtiles - 1 - pair) break;
    if (rep == 1 && only_rep < 0) __syncthreads();  // every wave is done with the first tile's LDS stages
    const int q0 = qt * F8_BR + w * 32;
    const int qi = q0 + l32;

    // A negative factor flips the sign bit of every Q code (exact); c > 0 afterwards.
    const bool neg = scale_log2 < 0.f;
    const float c = fmaxf(neg ? -scale_log2 : scale_log2, FLT_MIN);
    i32x8 qf[KK];
    if (qi < N) {
      const uint4* src = reinterpret_cast<const uint4*>(Q + q_base + (size_t)qi * HD);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[kk] = cat16(src[4 * kk + 2 * g], src[4 * kk + 2 * g + 1]);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[kk] = i32x8{};
    }
    // under a wave-uniform branch, outside the divergent row test
    if (neg) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[kk] ^= (int)0x80808080u;
    }

    const int q_end = min(N, qt * F8_BR + F8_BR);
    const int n_kt = CAUSAL ? (q_end + F8_BC - 1) / F8_BC : (N + F8_BC - 1) / F8_BC;

    // Direct-to-LDS staging: wave w issues blocks w, w + 4, ... of a tile (RPI rows each); lane i
    // fills row RPI * blk + i / CHUNKS at chunk position i % CHUNKS with the global chunk position
    // ^ swz(row). Rows past the sequence end fall outside the buffer resource and load as zeros.
    const int BLK_BYTES = 4 * RPI * HD;
    const int st_row = w * RPI + lane / CHUNKS;
    const int k_voff = st_row * HD + (((lane % CHUNKS) ^ swz8_k<HD>(st_row)) * 16);
    const int v_voff = st_row * HD + (((lane % CHUNKS) ^ swz8_v<HD>(st_row)) * 16);
    const uint8_t* k_head = K + kv_base;
    const uint8_t* v_head = V + kv_base;
    auto tile_bytes = [&](int row0) { return min(N - row0, F8_BC) * HD; };
    auto issue_k = [&](int kt, int stage) {
      const int row0 = kt * F8_BC;
      const u32x4 rsrc = dma_rsrc(k_head + (size_t)row0 * HD, tile_bytes(row0));
#pragma unroll
      for (int u = 0; u < BLOCKS / 4; ++u)
        load_to_lds<16>(rsrc, k_voff + u * BLK_BYTES, &sm.k[stage][(u * 4 + w) * RPI * HD]);
    };
    auto issue_v = [&](int kt, int stage) {
      const int row0 = kt * F8_BC;
      const u32x4 rsrc = dma_rsrc(v_head + (size_t)row0 * HD, tile_bytes(row0));
#pragma unroll
      for (int u = 0; u < BLOCKS / 4; ++u)
        load_to_lds<16>(rsrc, v_voff + u * BLK_BYTES, &sm.v[stage][(u * 4 + w) * RPI * HD]);
    };

    // K A-operand (S^T block kb, d block kk): row 32kb + l32, chunks 4kk + 2g and 4kk + 2g + 1.
    const int k_lane = l32 * HD;
    const int k_t = swz8_k<HD>(l32);
    // V^T A-operand: source lane 2k + bsel of a 16-lane group points at key row 16j + v_row and
    // byte column 32cb + 16 * ((lane / 16) % 2) + 8 * bsel; the key rows' swizzle is a lane constant.
    const int v_k = (lane & 15) >> 1;
    const int v_row = 8 * (v_k >> 2) + 4 * g + (v_k & 3);
    const int v_lane = v_row * HD + 8 * (lane & 1);
    const int v_c = (lane >> 4) & 1;
    const int v_t = swz8_v<HD>(v_row);

    // S^T for one tile, one 32-key block kb at a time: rows = keys 32kb + 8(r/4) + 4g + r%4,
    // column = this lane's query.
    auto scores_half = [&](const uint8_t* kbuf, f32x16 (&s)[2], int kb) {
      const uint8_t* krow = kbuf + 32 * kb * HD + k_lane;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(krow + (((4 * kk + 2 * g) ^ k_t) * 16));
        const uint4 a1 = *reinterpret_cast<const uint4*>(krow + (((4 * kk + 2 * g + 1) ^ k_t) * 16));
        s[kb] = mfma_f8(cat16(a0, a1), qf[kk], kk == 0 ? f32x16{} : s[kb]);
      }
    };
    auto scores = [&](const uint8_t* kbuf, f32x16 (&s)[2]) {
      scores_half(kbuf, s, 0);
      scores_half(kbuf, s, 1);
    };

    f32x16 oacc[CBLK];
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
    float m_run = -INFINITY;  // reference maximum (log2 units) shared by numerator and normaliser
    float l_run = 0.f;        // the normaliser of this lane's query (P carries the factor 2^6)

    // Slot (kb, r) holds key k0 + 4g + off(kb, r), off a compile-time constant below 64: a key is kept
    // when it is at most the lane's last visible key (one compare and one select per score).
    auto apply_mask = [&](int k0, f32x16 (&s)[2]) {
      const int last_key = CAUSAL ? min(qi, N - 1) : N - 1;
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

    // Online-softmax step on raw scores, in two parts around the (rare) output rescale. decide:
    // the tile maximum, the reference maximum and alpha; returns whether any lane of the wave raised
    // its reference (the caller then rescales the output accumulator).
    auto decide = [&](f32x16 (&s)[2], float& alpha) {
      float m1[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        const int a = 3 * i, bb = 3 * i + 1, c3 = 3 * i + 2;
        m1[i] = vmax3(s[a >> 4][a & 15], s[bb >> 4][bb & 15], s[c3 >> 4][c3 & 15]);
      }
      m1[10] = __builtin_elementwise_maximum(s[1][14], s[1][15]);
      const float m2a = vmax3(m1[0], m1[1], m1[2]), m2b = vmax3(m1[3], m1[4], m1[5]);
      const float m2c = vmax3(m1[6], m1[7], m1[8]), m2d = __builtin_elementwise_maximum(m1[9], m1[10]);
      const float rmax = vmax3(m2a, m2b, __builtin_elementwise_maximum(m2c, m2d));
      const float tmax = pair_max8(rmax) * c;
      const bool raise = tmax > m_run + kLazy;
      const float m_new = raise ? tmax : m_run;
      alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      return __builtin_amdgcn_ballot_w64(raise) != 0;
    };
    // probs: P^T as E4M3 codes in the B-operand byte order (byte 16kb + r <- accumulator s[kb][r]).
    auto probs = [&](const f32x16 (&s)[2], i32x8& pf) {
      const float bias = kPOffset - m_run;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kb = i >> 2, r0 = 4 * (i & 3);
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(s[kb][r0 + e], c, bias));
        // The low-half conversion leaves the high half of its register as it was, and the high-half
        // conversion then writes it, so any value may fill it: p[0]'s own bits let the conversion
        // write in place over p[0] (a zero there costs one move per word).
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], __float_as_int(p[0]), false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], word, true);
        pf[i] = word;
      }
    };
    // The tile's sum of the E4M3 probabilities of this lane's query, as the product of an all-ones
    // 32 x 64 block (E4M3 1.0 = 0x38) with P^T; every element of the result holds the column sum,
    // so element 0 is taken. The conversion does not saturate: a probability above 464 becomes the
    // E4M3 NaN code, and the matrix unit carries it into its query's sum (both measured on gfx950).
    // The all-ones operand is built once and made opaque to the compiler, which otherwise rebuilds
    // the constant before every use (eight moves per tile and wave).
    const int one4 = 0x38383838;
    i32x8 ones = {one4, one4, one4, one4, one4, one4, one4, one4};
    asm volatile("" : "+v"(ones));
    auto colsum = [&](const i32x8& pf) { return mfma_f8(ones, pf, f32x16{})[0]; };

    // O^T += V^T P^T: one 64-key MFMA per 32 output columns.
    auto pv = [&](const uint8_t* vbuf, const i32x8& pf) {
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        const uint8_t* vp = vbuf + v_lane + (((2 * cb + v_c) ^ v_t) * 16);
        i32x8 va;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const i32x2 t = lds_read_tr8(vp + 16 * j * HD);
          va[2 * j] = t[0];
          va[2 * j + 1] = t[1];
        }
        oacc[cb] = mfma_f8(va, pf, oacc[cb]);
      }
    };

    auto is_boundary = [&](int kt) {
      const int k0 = kt * F8_BC;
      return (k0 + F8_BC > N) || (CAUSAL && k0 + F8_BC - 1 > q0);
    };

    issue_k(0, 0);
    issue_v(0, 0);
    if (n_kt > 1) issue_k(1, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 s_cur[2];
    scores(sm.k[0], s_cur);
    __syncthreads();  // every wave has read K0 before its stage is reused for K2

    // Online-softmax step of tile kt. The probabilities are first taken against the current
    // reference, and while every one of them stays finite in E4M3 (no column sum is NaN) that
    // reference serves: no maximum, no rescale. Otherwise (a probability above 464, the reference
    // still unset, or a NaN score) the exact step runs: tile maximum, the lazy raise decision,
    // rescale of O, probabilities again. Every reference is some tile's maximum, at most the row's
    // maximum, and every probability that multiplies V is a finite E4M3 value at most 448.
    // Entering step kt: sc = S^T of tile kt, K_{kt+1} and V_kt in LDS. Issues V_{kt+1} and K_{kt+2},
    // the score MFMAs of tile kt+1 beside the softmax of tile kt, then O += V_kt P_kt.
    auto step = [&](int kt, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
      issue_v(kt + 1, (kt + 1) & 1);
      if (kt + 2 < n_kt) issue_k(kt + 2, kt & 1);
      if (is_boundary(kt)) apply_mask(kt * F8_BC, sc);
      i32x8 pf;
      // The first half of tile kt+1's score MFMAs goes with the exponentials, the second half
      // after the (rare) exact branch, then O += V P.
      scores_half(sm.k[(kt + 1) & 1], sn, 0);
      probs(sc, pf);
      float cs = colsum(pf);
      float alpha = 1.f;
      if (__builtin_amdgcn_ballot_w64(__builtin_isnan(cs)) != 0) {
        if (decide(sc, alpha)) {
#pragma unroll
          for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
        }
        probs(sc, pf);
        cs = colsum(pf);
      }
      scores_half(sm.k[(kt + 1) & 1], sn, 1);
      l_run = fmaf(l_run, alpha, cs);
      pv(sm.v[kt & 1], pf);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    auto last = [&](int kt, f32x16 (&sc)[2]) {
      if (is_boundary(kt)) apply_mask(kt * F8_BC, sc);
      i32x8 pf;
      probs(sc, pf);
      float cs = colsum(pf);
      float alpha = 1.f;
      if (__builtin_amdgcn_ballot_w64(__builtin_isnan(cs)) != 0) {
        if (decide(sc, alpha)) {
#pragma unroll
          for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
        }
        probs(sc, pf);
        cs = colsum(pf);
      }
      l_run = fmaf(l_run, alpha, cs);
      pv(sm.v[kt & 1], pf);
    };
    f32x16 s_alt[2];
    int kt = 0;
    for (; kt + 2 < n_kt; kt += 2) {
      step(kt, s_cur, s_alt);
      step(kt + 1, s_alt, s_cur);
    }
    // One last() on one buffer (two inlined copies cost registers around the exact branch).
    if (kt + 1 < n_kt) {
      step(kt, s_cur, s_alt);
      s_cur[0] = s_alt[0];
      s_cur[1] = s_alt[1];
      ++kt;
    }
    last(kt, s_cur);
    // The output accumulators are complete here, before the lane-divergent store below: left to
    // itself the compiler sinks the last tile's O += V P into that branch, where the matrix
    // instruction runs with the rows past N switched off in EXEC and returns wrong sums for the
    // other rows of the wave (measured).
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) asm volatile("" : "+v"(oacc[cb]));

    if (qi < N) {
      const float inv = v_descale / l_run;
      bf16* orow = O + q_base + (size_t)qi * HD;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          bf16x4 t = {to_bf16(oacc[cb][4 * rg + 0] * inv), to_bf16(oacc[cb][4 * rg + 1] * inv),
                      to_bf16(oacc[cb][4 * rg + 2] * inv), to_bf16(oacc[cb][4 * rg + 3] * inv)};
          *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * rg + 4 * g) = t;
        }
      }
      if (LSE != nullptr && g == 0) LSE[lse_base + qi] = (m_run - kPOffset + log2f(l_run)) * kLn2;
    }
  }
}

template <int HD, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
                  float scale_log2, float v_descale, hipStream_t stream, const char* name) {
  const int n_qt = (N + F8_BR - 1) / F8_BR;
  long long total = (long long)(CAUSAL ? (n_qt + 1) / 2 : n_qt) * H * B;
  // A causal grid of pairs that fills fewer than two workgroups per CU runs each pair as two
  // workgroups, as the bf16 forward does.
  const int cus = device_cus();
  const int split = CAUSAL && cus > 0 && total < 2LL * cus ? 1 : 0;
  if (split) total *= 2;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  TimedScope ts(name, stream);
  hipLaunchKernelGGL((fwd_fp8_kernel<HD, CAUSAL>), dim3((unsigned)total), dim3(F8_THREADS), 0, stream,
                     static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v),
                     static_cast<bf16*>(o), lse, H, H / H_kv, N, n_qt, scale_log2, v_descale, split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                          int N, int d, bool causal, float scale, float q_descale, float k_descale, float v_descale,
                          hipStream_t stream) {
  const float scale_log2 = (float)((double)scale * (double)q_descale * (double)k_descale * 1.4426950408889634);
  if (d == 128)
    return causal ? launch<128, true>(q, k, v, o, lse, B, H, H_kv, N, scale_log2, v_descale, stream,
                                      "fwd_fp8_d128_causal")
                  : launch<128, false>(q, k, v, o, lse, B, H, H_kv, N, scale_log2, v_descale, stream, "fwd_fp8_d128");
  return causal ? launch<64, true>(q, k, v, o, lse, B, H, H_kv, N, scale_log2, v_descale, stream, "fwd_fp8_d64_causal")
                : launch<64, false>(q, k, v, o, lse, B, H, H_kv, N, scale_log2, v_descale, stream, "fwd_fp8_d64");
}

}  // namespace ra
