// Attention backward for bf16 inputs on gfx950: dQ, dK, dV with no atomics.
//
// The scores are recomputed from Q and K ("Why Fast GPUs Still Wait for Memory", section
// "FlashAttention is an IO algorithm": the backward does more arithmetic because S is recomputed
// rather than stored), using the row log-sum-exp saved by the forward pass. Every gradient
// element is owned by exactly one workgroup, so no accumulation needs atomics: the race-free
// construction the MoA paper ("Validating Memory-Optimal Transformer Kernels on Real Hardware",
// sections 4.4-4.5) found decisive, where atomic accumulation doubled the kernel time. The price
// is recomputing S and dP in both the key-major and the query-major kernel; persisting dS instead
// doubled DRAM traffic in the same paper (section 4.7).
//
// Kernels, per (batch, head):
//   bwd_pre : D_i = sum_t dO[i,t] * O[i,t]   (equals sum_j P_ij dP_ij)
//   bwd_dkdv: workgroup = 128 keys (4 waves x 32); loops over 32-query tiles:
//             S = Q K^T, P = 2^(S*scale*log2e - LSE*log2e), dV += P^T dO, dP = dO V^T,
//             dS = P (dP - D), dK += dS^T Q; stores dK * scale and dV.
//   bwd_dq  : workgroup = 128 queries (4 waves x 32); loops over 64-key tiles:
//             S^T = K Q^T, P^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T;
//             stores dQ * scale.
// MFMA v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS are rounded to bf16 (nearest
// even) as MFMA operands. Operands whose contraction index is the row index of a stored tile are
// read from a transposed LDS copy made when the tile is staged.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ra {
namespace {

constexpr int BWD_THREADS = 256;

// ------------------------------------------------------------------------- preprocess ----

template <int HD>
__global__ __launch_bounds__(BWD_THREADS) void bwd_pre_kernel(const bf16* __restrict__ O,
                                                              const bf16* __restrict__ dO,
                                                              float* __restrict__ D, long long rows) {
  constexpr int CH = HD / 8;
  constexpr int RPB = BWD_THREADS / CH;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / CH;
  const int c = threadIdx.x % CH;
  float x = 0.f;
  if (row < rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(O + row * HD + c * 8);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + row * HD + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) x = fmaf(to_f32(a[e]), to_f32(g[e]), x);
  }
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));
  if constexpr (CH == 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true));
  if (row < rows && c == 0) D[row] = x;
}

// Stages a [32 rows x HD] bf16 tile into a row-major copy (stride HD + 8) and, optionally, a
// transposed copy (stride 32 + 4 per head-dimension row). Rows at or beyond n_rows are zero.
template <int HD, bool TRANSPOSED>
__device__ __forceinline__ void stage_rows32(const bf16* __restrict__ src, int row0, int n_rows,
                                             bf16* rm, bf16* tr, int tid) {
  constexpr int CH = HD / 8;
  constexpr int R = HD / 64;  // rows per thread (32 * CH / 256)
  const int cc = tid % CH;
  const int rg = tid / CH;
  bf16x8 x[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int row = rg * R + u;
    x[u] = row0 + row < n_rows ? *reinterpret_cast<const bf16x8*>(src + (size_t)(row0 + row) * HD + cc * 8)
                               : bf16x8{};
    *reinterpret_cast<bf16x8*>(rm + row * (HD + 8) + cc * 8) = x[u];
  }
  if constexpr (TRANSPOSED) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      bf16* dst = tr + (cc * 8 + e) * (32 + 4) + rg * R;
      if constexpr (R == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<bf16x2*>(dst) = bf16x2{x[0][e], x[1][e]};
      } else {
        dst[0] = x[0][e];
      }
    }
  }
}

// ------------------------------------------------------------------------------ dK dV ----

template <int HD>
struct DkdvSmem {
  bf16 q[32 * (HD + 8)];
  bf16 qt[HD * 36];
  bf16 dO[32 * (HD + 8)];
  bf16 dOt[HD * 36];
  float lse2[32];
  float Dv[32];
};

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(BWD_THREADS, 2) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dg,
    float* __restrict__ dK, float* __restrict__ dV, int H, int N, int n_ktiles, float scale,
    float scale_log2) {
  __shared__ DkdvSmem<HD> sm;
  constexpr int KSTEPS = HD / 16;
  constexpr int CBLK = HD / 32;
  constexpr int QS = HD + 8;

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  int kt = item % n_ktiles;
  const int bh = item / n_ktiles;
  if (CAUSAL) kt = n_ktiles - 1 - kt;  // (causal) low key tiles carry the most query tiles
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const size_t head = (size_t)bh * N * HD;
  const size_t rowbase = (size_t)bh * N;
  const int kw0 = kt * 128 + w * 32;  // this wave's first key
  const int key = kw0 + l32;          // B-operand column owned by this lane

  bf16x8 kf[KSTEPS], vf[KSTEPS];
  if (key < N) {
    const bf16x8* ks = reinterpret_cast<const bf16x8*>(K + head + (size_t)key * HD);
    const bf16x8* vs = reinterpret_cast<const bf16x8*>(V + head + (size_t)key * HD);
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

  const int n_qt = (N + 31) / 32;
  const int first_qt = CAUSAL ? (kt * 128) / 32 : 0;
  for (int qt = first_qt; qt < n_qt; ++qt) {
    const int i0 = qt * 32;
    __syncthreads();
    stage_rows32<HD, true>(Q + head, i0, N, sm.q, sm.qt, tid);
    stage_rows32<HD, true>(dO + head, i0, N, sm.dO, sm.dOt, tid);
    if (tid < 32) {
      const int i = i0 + tid;
      sm.lse2[tid] = i < N ? LSE[rowbase + i] * kLog2e : INFINITY;
      sm.Dv[tid] = i < N ? Dg[rowbase + i] : 0.f;
    }
    __syncthreads();
    if (CAUSAL && i0 + 31 < kw0) continue;  // every query of the tile precedes every key of the wave
    if (kw0 >= N) continue;

    // S and dP: lane column = key, rows = queries i0 + 8(r/4) + 4g + r%4.
    f32x16 s = f32x16{}, dp = f32x16{};
    const bf16* qrow = &sm.q[l32 * QS + 8 * g];
    const bf16* drow = &sm.dO[l32 * QS + 8 * g];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      s = mfma32(*reinterpret_cast<const bf16x8*>(qrow + 16 * kk), kf[kk], s);
      dp = mfma32(*reinterpret_cast<const bf16x8*>(drow + 16 * kk), vf[kk], dp);
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int il = 8 * (r >> 2) + 4 * g + (r & 3);
      const int i = i0 + il;
      const bool ok = key < N && (!CAUSAL || key <= i);  // rows i >= N have lse2 = +inf -> P = 0
      const float p = ok ? fast_exp2(s[r] * scale_log2 - sm.lse2[il]) : 0.f;
      const float ds = p * (dp[r] - sm.Dv[il]);
      pb[r >> 3][r & 7] = to_bf16(p);
      dsb[r >> 3][r & 7] = to_bf16(ds);
    }
    // dV += P^T dO and dK += dS^T Q. A operand: lane row = key, k-step hh covers queries
    // 16hh + {4g..4g+3, 8+4g..8+4g+3}; B operand: column c = 32cb + l32 from the transposed tile.
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        const bf16* dt = &sm.dOt[(32 * cb + l32) * 36 + 16 * hh + 4 * g];
        const bf16* qq = &sm.qt[(32 * cb + l32) * 36 + 16 * hh + 4 * g];
        const bf16x8 bdo = __builtin_shufflevector(*reinterpret_cast<const bf16x4*>(dt),
                                                   *reinterpret_cast<const bf16x4*>(dt + 8), 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 bq = __builtin_shufflevector(*reinterpret_cast<const bf16x4*>(qq),
                                                  *reinterpret_cast<const bf16x4*>(qq + 8), 0, 1, 2, 3, 4, 5, 6, 7);
        dv[cb] = mfma32(pb[hh], bdo, dv[cb]);
        dk[cb] = mfma32(dsb[hh], bq, dk[cb]);
      }
    }
  }

  // dK/dV accumulators: lane column c = 32cb + l32, rows = keys kw0 + 8(r/4) + 4g + r%4.
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (kr < N) {
        dK[head + (size_t)kr * HD + 32 * cb + l32] = dk[cb][r] * scale;
        dV[head + (size_t)kr * HD + 32 * cb + l32] = dv[cb][r];
      }
    }
  }
}

// --------------------------------------------------------------------------------- dQ ----

template <int HD>
struct DqSmem {
  bf16 k[64 * (HD + 8)];
  bf16 kt[HD * 68];
  bf16 v[64 * (HD + 8)];
};

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(BWD_THREADS, 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dg,
    float* __restrict__ dQ, int H, int N, int n_qtiles, float scale, float scale_log2) {
  __shared__ DqSmem<HD> sm;
  constexpr int KSTEPS = HD / 16;
  constexpr int CBLK = HD / 32;
  constexpr int KS = HD + 8;
  constexpr int CH = HD / 8;
  constexpr int LOADS = 64 * CH / BWD_THREADS;  // 16-byte chunks per thread per tile (K or V)

  const int item = xcd_remap(blockIdx.x, gridDim.x);
  int qt = item % n_qtiles;
  const int bh = item / n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int g = lane >> 5;

  const size_t head = (size_t)bh * N * HD;
  const size_t rowbase = (size_t)bh * N;
  const int q0 = qt * 128 + w * 32;
  const int qi = q0 + l32;

  bf16x8 qf[KSTEPS], df[KSTEPS];
  float lse2 = INFINITY, Dq = 0.f;
  if (qi < N) {
    const bf16x8* qs = reinterpret_cast<const bf16x8*>(Q + head + (size_t)qi * HD);
    const bf16x8* ds = reinterpret_cast<const bf16x8*>(dO + head + (size_t)qi * HD);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qf[kk] = qs[2 * kk + g];
      df[kk] = ds[2 * kk + g];
    }
    lse2 = LSE[rowbase + qi] * kLog2e;
    Dq = Dg[rowbase + qi];
  } else {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = df[kk] = bf16x8{};
  }

  f32x16 acc[CBLK];
#pragma unroll
  for (int cb = 0; cb < CBLK; ++cb) acc[cb] = f32x16{};

  const int q_end = min(N, qt * 128 + 128);
  const int n_kt = CAUSAL ? (q_end + 63) / 64 : (N + 63) / 64;
  const int vc = tid % CH;
  const int vg = tid / CH;  // LOADS consecutive keys per thread for the transposed K copy
  for (int t = 0; t < n_kt; ++t) {
    const int k0 = t * 64;
    __syncthreads();
    {
      bf16x8 kx[LOADS];
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int c = tid + BWD_THREADS * u;
        const int row = c / CH;
        const int col = c % CH;
        const bool in = k0 + row < N;
        const bf16x8 kv = in ? *reinterpret_cast<const bf16x8*>(K + head + (size_t)(k0 + row) * HD + col * 8) : bf16x8{};
        const bf16x8 vv = in ? *reinterpret_cast<const bf16x8*>(V + head + (size_t)(k0 + row) * HD + col * 8) : bf16x8{};
        *reinterpret_cast<bf16x8*>(&sm.k[row * KS + col * 8]) = kv;
        *reinterpret_cast<bf16x8*>(&sm.v[row * KS + col * 8]) = vv;
        const int krow = vg * LOADS + u;
        kx[u] = k0 + krow < N ? *reinterpret_cast<const bf16x8*>(K + head + (size_t)(k0 + krow) * HD + vc * 8)
                              : bf16x8{};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16* dst = &sm.kt[(vc * 8 + e) * 68 + vg * LOADS];
        if constexpr (LOADS == 4) {
          *reinterpret_cast<bf16x4*>(dst) = bf16x4{kx[0][e], kx[1][e], kx[2][e], kx[3][e]};
        } else {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          *reinterpret_cast<bf16x2*>(dst) = bf16x2{kx[0][e], kx[1][e]};
        }
      }
    }
    __syncthreads();

    bool need[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) need[kb] = (k0 + 32 * kb < N) && (!CAUSAL || k0 + 32 * kb <= q0 + 31);

    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
      if (need[kb]) {
        const bf16* krow = &sm.k[(32 * kb + l32) * KS + 8 * g];
        const bf16* vrow = &sm.v[(32 * kb + l32) * KS + 8 * g];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          s = mfma32(*reinterpret_cast<const bf16x8*>(krow + 16 * kk), qf[kk], s);
          dp = mfma32(*reinterpret_cast<const bf16x8*>(vrow + 16 * kk), df[kk], dp);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = k0 + 32 * kb + 8 * (r >> 2) + 4 * g + (r & 3);
        const bool ok = need[kb] && kr < N && (!CAUSAL || kr <= qi);
        const float p = ok ? fast_exp2(s[r] * scale_log2 - lse2) : 0.f;
        dsb[2 * kb + (r >> 3)][r & 7] = to_bf16(p * (dp[r] - Dq));
      }
    }
    // dQ^T += K^T dS^T: A operand = K^T row c = 32cb + l32, keys 32kb + 16hh + {4g.., 8+4g..}.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kb = ks >> 1;
      const int hh = ks & 1;
      if (!need[kb]) continue;
#pragma unroll
      for (int cb = 0; cb < CBLK; ++cb) {
        const bf16* kr = &sm.kt[(32 * cb + l32) * 68 + 32 * kb + 16 * hh + 4 * g];
        const bf16x8 a = __builtin_shufflevector(*reinterpret_cast<const bf16x4*>(kr),
                                                 *reinterpret_cast<const bf16x4*>(kr + 8), 0, 1, 2, 3, 4, 5, 6, 7);
        acc[cb] = mfma32(a, dsb[ks], acc[cb]);
      }
    }
  }

  if (qi < N) {
    float* out = dQ + head + (size_t)qi * HD;
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

template <int HD, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, float scale,
                  void* ws, hipStream_t stream, const char* pre_name, const char* dkdv_name,
                  const char* dq_name) {
  const bf16* Q = static_cast<const bf16*>(q);
  const bf16* K = static_cast<const bf16*>(k);
  const bf16* V = static_cast<const bf16*>(v);
  const bf16* O = static_cast<const bf16*>(o);
  const bf16* dO = static_cast<const bf16*>(dout);
  float* D = static_cast<float*>(ws);
  const long long rows = (long long)B * H * N;
  constexpr int RPB = BWD_THREADS / (HD / 8);
  {
    TimedScope ts(pre_name, stream);
    hipLaunchKernelGGL((bwd_pre_kernel<HD>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(BWD_THREADS), 0,
                       stream, O, dO, D, rows);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_t = (N + 127) / 128;
  const unsigned total = (unsigned)((long long)n_t * H * B);
  {
    TimedScope ts(dkdv_name, stream);
    hipLaunchKernelGGL((bwd_dkdv_kernel<HD, CAUSAL>), dim3(total), dim3(BWD_THREADS), 0, stream, Q, K, V, dO,
                       lse, D, dk, dv, H, N, n_t, scale, scale * kLog2e);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    TimedScope ts(dq_name, stream);
    hipLaunchKernelGGL((bwd_dq_kernel<HD, CAUSAL>), dim3(total), dim3(BWD_THREADS), 0, stream, Q, K, V, dO, lse,
                       D, dq, H, N, n_t, scale, scale * kLog2e);
  }
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  return (size_t)B * H * N * sizeof(float);
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                      bool causal, float scale, void* ws, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch<128, true>(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, scale, ws, stream,
                                      "bwd_pre_d128", "bwd_dkdv_d128_causal", "bwd_dq_d128_causal")
                  : launch<128, false>(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, scale, ws, stream,
                                       "bwd_pre_d128", "bwd_dkdv_d128", "bwd_dq_d128");
  }
  return causal ? launch<64, true>(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, scale, ws, stream,
                                   "bwd_pre_d64", "bwd_dkdv_d64_causal", "bwd_dq_d64_causal")
                : launch<64, false>(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, scale, ws, stream,
                                    "bwd_pre_d64", "bwd_dkdv_d64", "bwd_dq_d64");
}

}  // namespace ra
