// Fused tiled attention forward for bf16 inputs on gfx950 (MFMA 32x32x16 bf16, fp32 accumulate).
//
// Schedule ("Why Fast GPUs Still Wait for Memory", section "FlashAttention is an IO algorithm"):
// a workgroup owns FWD_BR query rows of one (batch, head); it streams every K/V tile of FWD_BC
// keys through LDS, keeps a running row maximum and normaliser, rescales its output accumulator
// as each tile arrives, and never writes S or P to memory. Causal workgroups stop at the
// diagonal and mask only the tiles that straddle it (same page, note on causal masking).
//
// gfx950 mapping:
//   * 4 waves x 32 query rows. Each wave keeps its Q rows in registers as the MFMA B operand.
//   * Scores are produced transposed, S^T = K Q^T (A = K rows from LDS, B = Q), so that each lane
//     holds one query row: the row max/sum need one cross-lane exchange (lane ^ 32) and the
//     probabilities leave the accumulator already in the B-operand layout of O^T = V^T P^T.
//   * V is stored transposed in LDS (V^T[d][key]) when the tile is staged, so the A operand of
//     O^T = V^T P^T is two 8-byte LDS reads per MFMA.
//   * The next tile is prefetched into registers while the current one is consumed.
//   * Workgroup ids are remapped so the query tiles of one head run on one XCD (shared L2), and
//     causal tiles run heaviest first to shorten the tail.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ra {
namespace {

constexpr int FWD_BR = 128;
constexpr int FWD_BC = 64;
constexpr int FWD_THREADS = 256;

template <int HD>
struct FwdSmem {
  static constexpr int KSTR = HD + 8;      // bf16 per K row (16-byte pad skews LDS banks)
  static constexpr int VSTR = FWD_BC + 4;  // bf16 per V^T row (8-byte pad)
  bf16 k[FWD_BC * KSTR];
  bf16 vt[HD * VSTR];
};

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(FWD_THREADS, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int H, int group, int N, int n_qtiles,
    float scale_log2) {
  __shared__ FwdSmem<HD> sm;
  constexpr int KSTR = FwdSmem<HD>::KSTR;
  constexpr int VSTR = FwdSmem<HD>::VSTR;
  constexpr int KSTEPS = HD / 16;  // MFMA k-steps over the head dimension
  constexpr int CBLK = HD / 32;    // 32-wide head-dimension blocks of O^T
  constexpr int CHUNKS = HD / 8;   // 16-byte chunks per row
  constexpr int LOADS = FWD_BC * CHUNKS / FWD_THREADS;  // 16-byte loads per thread per tile
  constexpr int VKEYS = LOADS;     // consecutive keys per thread in the V^T store

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

  bf16x8 qf[KSTEPS];
  if (qi < N) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(Q + q_head + (size_t)qi * HD);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = src[2 * kk + g];
  } else {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = bf16x8{};
  }

  const int q_end = min(N, qt * FWD_BR + FWD_BR);
  const int n_kt = CAUSAL ? (q_end + FWD_BC - 1) / FWD_BC : (N + FWD_BC - 1) / FWD_BC;

  // Per-thread staging assignment. K: chunk c = tid + 256u -> (row c / CHUNKS, col c % CHUNKS).
  // V: chunk column vc, VKEYS consecutive keys starting at vg * VKEYS.
  const int vc = tid % CHUNKS;
  const int vg = tid / CHUNKS;

  bf16x8 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int kt) {
    const int k0 = kt * FWD_BC;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + FWD_THREADS * u;
      const int key = k0 + c / CHUNKS;
      kreg[u] = key < N ? *reinterpret_cast<const bf16x8*>(K + kv_head + (size_t)key * HD + (c % CHUNKS) * 8)
                        : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int key = k0 + vg * VKEYS + u;
      vreg[u] = key < N ? *reinterpret_cast<const bf16x8*>(V + kv_head + (size_t)key * HD + vc * 8)
                        : bf16x8{};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + FWD_THREADS * u;
      *reinterpret_cast<bf16x8*>(&sm.k[(c / CHUNKS) * KSTR + (c % CHUNKS) * 8]) = kreg[u];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16* dst = &sm.vt[(vc * 8 + e) * VSTR + vg * VKEYS];
      if constexpr (VKEYS == 4) {
        bf16x4 t = {vreg[0][e], vreg[1][e], vreg[2][e], vreg[3][e]};
        *reinterpret_cast<bf16x4*>(dst) = t;
      } else {
        static_assert(VKEYS == 2, "tile geometry");
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 t = {vreg[0][e], vreg[1][e]};
        *reinterpret_cast<bf16x2*>(dst) = t;
      }
    }
  };

  f32x16 oacc[CBLK];
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) oacc[cb] = f32x16{};
  float m_run = -INFINITY;  // running max of scale*log2(e)*s for this lane's query row
  float l_run = 0.f;        // this lane's share of the running normaliser

  load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();  // all waves are done with the previous tile
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(kt + 1);

    const int k0 = kt * FWD_BC;
    bool need[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      need[kb] = (k0 + 32 * kb < N) && (!CAUSAL || k0 + 32 * kb <= q0 + 31);

    // S^T block kb: rows = keys k0 + 32kb + (8(r/4) + 4g + r%4), column = this lane's query.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      if (need[kb]) {
        const bf16* krow = &sm.k[(32 * kb + l32) * KSTR + 8 * g];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 16 * kk);
          s[kb] = mfma32(kf, qf[kk], s[kb]);
        }
      }
    }

    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = need[kb] && key < N && (!CAUSAL || key <= qi);
        const float x = ok ? s[kb][r] * scale_log2 : -INFINITY;
        s[kb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
    // Tile 0 always holds key 0, which every query row keeps, so m_new is finite from the start.
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < CBLK; ++cb) oacc[cb] *= alpha;

    // P^T in the B-operand layout: k-step ks = 2kb + hh takes accumulator slots 8hh .. 8hh+7.
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(s[kb][r] - m_new);
        l_run += p;
        pf[2 * kb + (r >> 3)][r & 7] = to_bf16(p);
      }
    }

    // O^T += V^T P^T. A operand: V^T row (32cb + l32), keys 32kb + 16hh + {4g..4g+3, 8+4g..8+4g+3}.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1;
      const int hh = ks & 1;
      if (!need[kb]) continue;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        const bf16* vrow = &sm.vt[(32 * cb + l32) * VSTR + 32 * kb + 16 * hh + 4 * g];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
        const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[cb] = mfma32(va, pf[ks], oacc[cb]);
      }
    }
  }

  l_run += shfl_xor_f(l_run, 32);
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
