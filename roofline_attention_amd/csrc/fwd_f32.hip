// Fused tiled attention forward for float32 storage and arithmetic (the tight-tolerance path).
//
// Same schedule as the bf16 kernel ("Why Fast GPUs Still Wait for Memory", section
// "FlashAttention is an IO algorithm"): K/V tiles stream through LDS, S and P stay on chip, and a
// running maximum and normaliser rescale the output as each tile arrives. The arithmetic is plain
// fp32 FMA on the vector ALUs: two lanes own one query row, each holding half of the head
// dimension of q and of the output accumulator, and their partial dot products are joined with
// one DPP exchange. All lanes of a half read the same LDS word (a broadcast, no bank conflict).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ra {
namespace {

constexpr int F32_BR = 64;   // query rows per workgroup
constexpr int F32_BC = 32;   // keys per tile
constexpr int F32_THREADS = 2 * F32_BR;

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(F32_THREADS) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int H, int group, int N, int n_qtiles,
    float scale_log2) {
  constexpr int HALF = HD / 2;
  __shared__ float ks[F32_BC][HD];
  __shared__ float vs[F32_BC][HD];

  const int item = blockIdx.x;
  const int qt = item % n_qtiles;
  const int bh = item / n_qtiles;
  const int h = bh % H;
  const int b = bh / H;
  const int Hkv = H / group;
  const int hk = h / group;
  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int qi = qt * F32_BR + (tid >> 1);

  const size_t q_head = ((size_t)b * H + h) * (size_t)N * HD;
  const size_t kv_head = ((size_t)b * Hkv + hk) * (size_t)N * HD;

  float q[HALF], o[HALF];
#pragma unroll
  for (int e = 0; e < HALF; ++e) {
    q[e] = qi < N ? Q[q_head + (size_t)qi * HD + half * HALF + e] : 0.f;
    o[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  const int q_end = min(N, qt * F32_BR + F32_BR);
  const int n_kt = CAUSAL ? (q_end + F32_BC - 1) / F32_BC : (N + F32_BC - 1) / F32_BC;
  constexpr int VEC = F32_BC * HD / 4;  // float4 per tile

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * F32_BC;
    __syncthreads();
    for (int c = tid; c < VEC; c += F32_THREADS) {
      const int row = c / (HD / 4);
      const int col = (c % (HD / 4)) * 4;
      const int key = k0 + row;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (key < N) {
        kv = *reinterpret_cast<const float4*>(K + kv_head + (size_t)key * HD + col);
        vv = *reinterpret_cast<const float4*>(V + kv_head + (size_t)key * HD + col);
      }
      *reinterpret_cast<float4*>(&ks[row][col]) = kv;
      *reinterpret_cast<float4*>(&vs[row][col]) = vv;
    }
    __syncthreads();

    float s[F32_BC];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < F32_BC; ++j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < HALF; ++e) part = fmaf(q[e], ks[j][half * HALF + e], part);
      part += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(part), 0xB1, 0xF, 0xF, true));
      const int key = k0 + j;
      const bool ok = key < N && (!CAUSAL || key <= qi);
      s[j] = ok ? part * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m_run, tmax);  // finite: tile 0 holds key 0
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < HALF; ++e) o[e] *= alpha;
#pragma unroll
    for (int j = 0; j < F32_BC; ++j) {
      const float p = exp2f(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int e = 0; e < HALF; ++e) o[e] = fmaf(p, vs[j][half * HALF + e], o[e]);
    }
  }

  if (qi < N) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int e = 0; e < HALF; ++e) O[q_head + (size_t)qi * HD + half * HALF + e] = o[e] * inv;
    if (LSE != nullptr && half == 0) LSE[((size_t)b * H + h) * N + qi] = (m_run + log2f(l_run)) * kLn2;
  }
}

template <int HD, bool CAUSAL>
hipError_t launch(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H,
                  int H_kv, int N, float scale, hipStream_t stream, const char* name) {
  const int n_qt = (N + F32_BR - 1) / F32_BR;
  const long long total = (long long)n_qt * H * B;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  TimedScope ts(name, stream);
  hipLaunchKernelGGL((fwd_f32_kernel<HD, CAUSAL>), dim3((unsigned)total), dim3(F32_THREADS), 0, stream,
                     q, k, v, o, lse, H, H / H_kv, N, n_qt, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                          int H, int H_kv, int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch<128, true>(q, k, v, o, lse, B, H, H_kv, N, scale, stream, "fwd_f32_d128_causal")
                  : launch<128, false>(q, k, v, o, lse, B, H, H_kv, N, scale, stream, "fwd_f32_d128");
  }
  return causal ? launch<64, true>(q, k, v, o, lse, B, H, H_kv, N, scale, stream, "fwd_f32_d64_causal")
                : launch<64, false>(q, k, v, o, lse, B, H, H_kv, N, scale, stream, "fwd_f32_d64");
}

}  // namespace ra
