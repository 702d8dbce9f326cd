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
//   * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4, no VGPR staging),
//     double-buffered so the loads of tile j+1 overlap the math of tile j with one barrier per
//     tile. Each wave instruction fills 1 KB of LDS in lane order, so bank conflicts are avoided by
//     an XOR swizzle of the 16-byte chunks within a row instead of padding.
//   * The V^T operand of O^T = V^T P^T comes from ds_read_b64_tr_b16, which transposes 16-bit
//     elements across each 16-lane group, so V is never transposed in memory.
//   * The running maximum is only raised when a tile's maximum exceeds it by more than 8 (log2
//     units); the numerator and the normaliser always share the same reference, so the result is
//     unchanged while the output rescale is skipped on almost every tile.
//   * Masks are evaluated only on tiles that cross the causal diagonal or the sequence end.
//   * Workgroup ids are remapped so the query tiles of one head run on one XCD (shared L2), and
//     causal tiles run heaviest first to shorten the tail.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ra {
namespace {

constexpr int FWD_BR = 128;
constexpr int FWD_BC = 64;
constexpr int FWD_THREADS = 256;
constexpr float kLazyRescale = 8.0f;  // log2 units: P values stay below 2^8

// LDS tiles: [2 stages][FWD_BC rows][HD] bf16, unpadded. The 16-byte chunk c of row r is stored
// at chunk position c ^ swz(r): swz_k(r) = r mod CH spreads the 32 rows one MFMA A-operand read
// touches over all banks; swz_v(r) = 2r mod CH does the same for the 4-row x 32-byte footprint
// of a 16-lane transposed read.
template <int HD>
struct FwdSmem {
  bf16 k[2][FWD_BC * HD];
  bf16 v[2][FWD_BC * HD];
};

template <int HD>
__device__ __forceinline__ int swz_k(int r) { return r & (HD / 8 - 1); }
template <int HD>
__device__ __forceinline__ int swz_v(int r) { return (2 * r) & (HD / 8 - 1); }

typedef void __attribute__((address_space(3))) * lds_void_ptr;
typedef const void __attribute__((address_space(1))) * global_void_ptr;

// One 16-byte-per-lane direct load into LDS: lane i of the wave writes lds_block + 16 i.
__device__ __forceinline__ void load_to_lds(const void* src, void* lds_block) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)lds_block, 16, 0, 0);
}

typedef bf16x4 __attribute__((address_space(3))) * lds_bf16x4_ptr;

__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p));
}

// max over the lane pair (l, l ^ 32) that shares one query row
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(FWD_THREADS, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int H, int group, int N, int n_qtiles,
    float scale_log2) {
  __shared__ FwdSmem<HD> sm;
  constexpr int KSTEPS = HD / 16;  // MFMA k-steps over the head dimension
  constexpr int CBLK = HD / 32;    // 32-wide head-dimension blocks of O^T
  constexpr int CHUNKS = HD / 8;   // 16-byte chunks per row

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  int qt = item % n_qtiles;
  const int bh = item / n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int h = bh % H;
  const int b = bh / H;
  const int Hkv = H / group;
  const int hk = h / group;

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const size_t q_head = ((size_t)b * H + h) * (size_t)N * HD;
  const size_t kv_head = ((size_t)b * Hkv + hk) * (size_t)N * HD;
  const int q0 = qt * FWD_BR + w * 32;
  const int qi = q0 + l32;

  // A negative scale is folded into Q (exact sign flip) so the exponent factor is >= 0 and the
  // row maximum of the raw scores gives the maximum of the scaled ones.
  const bool neg = scale_log2 < 0.f;
  const float c = neg ? -scale_log2 : scale_log2;
  bf16x8 qf[KSTEPS];
  if (qi < N) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(Q + q_head + (size_t)qi * HD);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qf[kk] = src[2 * kk + g];
      if (neg) qf[kk] = -qf[kk];
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = bf16x8{};
  }

  const int q_end = min(N, qt * FWD_BR + FWD_BR);
  const int n_kt = CAUSAL ? (q_end + FWD_BC - 1) / FWD_BC : (N + FWD_BC - 1) / FWD_BC;

  // Direct-to-LDS staging: a wave instruction covers RPI rows (1 KB); wave w issues blocks
  // w, w + 4, ... of the tile. Lane i fills row blk*RPI + i / CHUNKS, chunk position i % CHUNKS,
  // with global chunk position ^ swz(row). Rows past the sequence end re-read row N-1 (finite
  // data; their scores are masked).
  constexpr int RPI = 1024 / (HD * 2);
  constexpr int BLOCKS = FWD_BC / RPI;  // wave instructions per tensor per tile
  auto issue_tile = [&](int kt, int stage) {
    const int k0 = kt * FWD_BC;
#pragma unroll
    for (int u = 0; u < BLOCKS / 4; ++u) {
      const int blk = u * 4 + w;
      const int row = blk * RPI + lane / CHUNKS;
      const int pos = lane % CHUNKS;
      const size_t grow = kv_head + (size_t)min(k0 + row, N - 1) * HD;
      load_to_lds(K + grow + ((pos ^ swz_k<HD>(row)) * 8), &sm.k[stage][blk * RPI * HD]);
      load_to_lds(V + grow + ((pos ^ swz_v<HD>(row)) * 8), &sm.v[stage][blk * RPI * HD]);
    }
  };

  // K A-operand read (S^T block kb, k-step kk): row 32kb + l32, chunk 2kk + g at position
  // (2kk + g) ^ swz_k(l32) (32kb is a multiple of CH rows' swizzle period).
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

  f32x16 oacc[CBLK];
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;  // reference maximum (log2 units) shared by numerator and normaliser
  float l_run = 0.f;        // this lane's share of the normaliser

  // One K/V tile. MASK selects the path that evaluates the causal / sequence-end masks.
  auto tile = [&](const int k0, const bf16* kbuf, const bf16* vbuf, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    bool need[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      need[kb] = !MASK || ((k0 + 32 * kb < N) && (!CAUSAL || k0 + 32 * kb <= q0 + 31));

    // S^T block kb: rows = keys k0 + 32kb + 8(r/4) + 4g + r%4, column = this lane's query.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      if (need[kb]) {
        const bf16* krow = &kbuf[32 * kb * HD + k_lane];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
          s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(krow + ((2 * kk) ^ k_t) * 8), qf[kk], s[kb]);
      }
    }

    float tmax;
    if constexpr (MASK) {
      tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
          const bool ok = need[kb] && key < N && (!CAUSAL || key <= qi);
          const float x = ok ? s[kb][r] * c : -INFINITY;  // scaled score, -inf where masked
          s[kb][r] = x;
          tmax = fmaxf(tmax, x);
        }
      }
    } else {
      float rmax = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) rmax = fmaxf(rmax, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) rmax = fmaxf(rmax, s[1][r]);
      tmax = rmax * c;
    }
    tmax = pair_max(tmax);
    // Tile 0 always holds key 0, which every query row keeps, so m_run is finite after it.
    const bool raise = tmax > m_run + kLazyRescale;
    const float m_new = raise ? tmax : m_run;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;
    }
    m_run = m_new;

    // P^T in the B-operand layout: k-step ks = 2kb + hh takes accumulator slots 8hh .. 8hh+7.
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = MASK ? fast_exp2(s[kb][r] - m_new) : fast_exp2(fmaf(s[kb][r], c, -m_new));
        l_run += p;
        pf[2 * kb + (r >> 3)][r & 7] = to_bf16(p);
      }
    }

    // O^T += V^T P^T. A operand: lane row c = 32cb + l32, keys 32kb + 16hh + {4g..4g+3, 8+4g..8+4g+3}.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1;
      const int hh = ks & 1;
      if (!need[kb]) continue;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        const bf16* vp = &vbuf[(32 * kb + 16 * hh) * HD + v_lane + ((4 * cb) ^ v_t) * 8];
        const bf16x8 va = __builtin_shufflevector(lds_read_tr(vp), lds_read_tr(vp + 8 * HD), 0, 1, 2, 3, 4, 5,
                                                  6, 7);
        oacc[cb] = mfma32(va, pf[ks], oacc[cb]);
      }
    }
  };

  issue_tile(0, 0);
  for (int kt = 0; kt < n_kt; ++kt) {
    // This wave's loads of tile kt have landed; after the barrier every wave's have, and every
    // wave has finished reading the stage that tile kt + 1 overwrites.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 1 < n_kt) issue_tile(kt + 1, (kt + 1) & 1);
    const int k0 = kt * FWD_BC;
    const bf16* kbuf = sm.k[kt & 1];
    const bf16* vbuf = sm.v[kt & 1];
    const bool boundary = (k0 + FWD_BC > N) || (CAUSAL && k0 + FWD_BC - 1 > q0);
    if (boundary)
      tile(k0, kbuf, vbuf, std::integral_constant<bool, true>{});
    else
      tile(k0, kbuf, vbuf, std::integral_constant<bool, false>{});
  }

  l_run += __shfl_xor(l_run, 32, 64);
  if (qi < N) {
    const float inv = 1.f / l_run;
    bf16* orow = O + q_head + (size_t)qi * HD;
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 t = {to_bf16(oacc[cb][4 * rg + 0] * inv), to_bf16(oacc[cb][4 * rg + 1] * inv),
                    to_bf16(oacc[cb][4 * rg + 2] * inv), to_bf16(oacc[cb][4 * rg + 3] * inv)};
        *reinterpret_cast<bf16x4*>(orow + 32 * cb + 8 * rg + 4 * g) = t;
      }
    }
    if (LSE != nullptr && g == 0) LSE[((size_t)b * H + h) * N + qi] = (m_run + log2f(l_run)) * kLn2;
  }
}

template <int HD, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int H_kv, int N, float scale, hipStream_t stream, const char* name) {
  const int n_qt = (N + FWD_BR - 1) / FWD_BR;
  const long long total = (long long)n_qt * H * B;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  TimedScope ts(name, stream);
  hipLaunchKernelGGL((fwd_bf16_kernel<HD, CAUSAL>), dim3((unsigned)total), dim3(FWD_THREADS), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                     static_cast<bf16*>(o), lse, H, H / H_kv, N, n_qt, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int H_kv, int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch<128, true>(q, k, v, o, lse, B, H, H_kv, N, scale, stream, "fwd_bf16_d128_causal")
                  : launch<128, false>(q, k, v, o, lse, B, H, H_kv, N, scale, stream, "fwd_bf16_d128");
  }
  return causal ? launch<64, true>(q, k, v, o, lse, B, H, H_kv, N, scale, stream, "fwd_bf16_d64_causal")
                : launch<64, false>(q, k, v, o, lse, B, H, H_kv, N, scale, stream, "fwd_bf16_d64");
}

}  // namespace ra
