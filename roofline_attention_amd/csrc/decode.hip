// Split-KV decode attention for one query token per (sequence, head) over a bf16 KV cache.
//
// Decode is memory-bound at I = 2g/s FLOP/byte for group size g ("Why Fast GPUs Still Wait for
// Memory", section "Attention III - KV cache, GQA, MLA"), so the kernel is built to stream K and V
// at HBM rate: every K/V byte is read once, and all g query heads of a KV head are served from
// the same bytes (the grouped physical path, no K/V expansion). The key axis is split into
// fixed-size chunks, one wave each, so ragged sequence lengths never leave a long serial tail;
// the partial (max, sum, output) triples are merged by a second kernel ("M4.2 - GPU Execution
// Model for Transformer Kernels", section 0x08: split-K trades parallelism for an extra
// reduction pass).
//
// Split kernel, one 64-lane wave per (split, KV head, sequence):
//   lane = (key slot ks, 16-byte chunk dc of the head dimension). One load instruction covers
//   KPI consecutive cache rows (contiguous bytes), the partial dot products are joined across the
//   chunk lanes with DPP, and the chunk's softmax is kept online over sub-chunks of ITERS * KPI
//   keys. The partial record of each query head is {m, l, -, -, o[d]} with m in log2 units of
//   the scaled score and o not yet divided by l.
// Combine kernel, one wave per (query head, sequence): M = max m_s, L = sum 2^(m_s - M) l_s,
//   O = sum 2^(m_s - M) o_s / L, LSE = ln 2 * (M + log2 L).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace ra {
namespace {

constexpr int DEC_ITERS = 8;  // key rows per lane-slot per sub-chunk

template <int CH>
__device__ __forceinline__ float chunk_sum(float x) {
  static_assert(CH == 16 || CH == 8, "chunk lanes");
  if constexpr (CH == 16) {
    return row16_sum(x);
  } else {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));
    return x;
  }
}

// Reduction across the key slots (lanes that differ in the bits above the chunk bits).
template <int CH>
__device__ __forceinline__ float slots_max(float x) {
#pragma unroll
  for (int m = CH; m < 64; m <<= 1) x = fmaxf(x, shfl_xor_f(x, m));
  return x;
}
template <int CH>
__device__ __forceinline__ float slots_sum(float x) {
#pragma unroll
  for (int m = CH; m < 64; m <<= 1) x += shfl_xor_f(x, m);
  return x;
}

__device__ __forceinline__ int clamp_len(const int32_t* kv_len, int b, int N_cap) {
  const int len = kv_len[b];
  return len < 0 ? 0 : (len > N_cap ? N_cap : len);
}

template <int HD, int G>
__global__ __launch_bounds__(64) void decode_split_kernel(
    const bf16* __restrict__ Qd, const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
    const int32_t* __restrict__ kv_len, float* __restrict__ ws, int H, int H_kv, int N_cap,
    int n_split, float scale_log2) {
  constexpr int CH = HD / 8;       // lanes per cache row (16-byte chunks)
  constexpr int KPI = 64 / CH;     // cache rows per load instruction
  constexpr int SUB = KPI * DEC_ITERS;
  constexpr int REC = HD + 4;

  const int split = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int len = clamp_len(kv_len, b, N_cap);
  const int k_begin = split * kDecodeSplit;
  if (k_begin >= len) return;
  const int k_end = min(len, k_begin + kDecodeSplit);

  const int lane = threadIdx.x;
  const int dc = lane % CH;
  const int ks = lane / CH;

  float qv[G][8];
#pragma unroll
  for (int hq = 0; hq < G; ++hq) {
    const bf16x8 t = *reinterpret_cast<const bf16x8*>(Qd + ((size_t)b * H + hk * G + hq) * HD + dc * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[hq][e] = to_f32(t[e]) * scale_log2;
  }

  const size_t head = ((size_t)b * H_kv + hk) * (size_t)N_cap * HD;
  const bf16* kbase = Kc + head + dc * 8;
  const bf16* vbase = Vc + head + dc * 8;

  float m_run[G], l_run[G], o[G][8];
#pragma unroll
  for (int hq = 0; hq < G; ++hq) {
    m_run[hq] = -INFINITY;
    l_run[hq] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hq][e] = 0.f;
  }

  for (int s0 = k_begin; s0 < k_end; s0 += SUB) {
    bf16x8 kr[DEC_ITERS], vr[DEC_ITERS];
#pragma unroll
    for (int it = 0; it < DEC_ITERS; ++it) {
      const int key = s0 + it * KPI + ks;
      kr[it] = key < k_end ? *reinterpret_cast<const bf16x8*>(kbase + (size_t)key * HD) : bf16x8{};
    }
#pragma unroll
    for (int it = 0; it < DEC_ITERS; ++it) {
      const int key = s0 + it * KPI + ks;
      vr[it] = key < k_end ? *reinterpret_cast<const bf16x8*>(vbase + (size_t)key * HD) : bf16x8{};
    }

    float s[DEC_ITERS][G];
#pragma unroll
    for (int it = 0; it < DEC_ITERS; ++it) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = to_f32(kr[it][e]);
      const bool ok = s0 + it * KPI + ks < k_end;
#pragma unroll
      for (int hq = 0; hq < G; ++hq) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(qv[hq][e], kf[e], acc);
        acc = chunk_sum<CH>(acc);
        s[it][hq] = ok ? acc : -INFINITY;
      }
    }

#pragma unroll
    for (int hq = 0; hq < G; ++hq) {
      float mx = s[0][hq];
#pragma unroll
      for (int it = 1; it < DEC_ITERS; ++it) mx = fmaxf(mx, s[it][hq]);
      mx = slots_max<CH>(mx);
      // The first sub-chunk holds key k_begin < k_end, so m_new is finite from the start.
      const float m_new = fmaxf(m_run[hq], mx);
      const float alpha = fast_exp2(m_run[hq] - m_new);
      m_run[hq] = m_new;
      l_run[hq] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hq][e] *= alpha;
    }

#pragma unroll
    for (int it = 0; it < DEC_ITERS; ++it) {
      float vf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) vf[e] = to_f32(vr[it][e]);
#pragma unroll
      for (int hq = 0; hq < G; ++hq) {
        const float p = fast_exp2(s[it][hq] - m_run[hq]);
        l_run[hq] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hq][e] = fmaf(p, vf[e], o[hq][e]);
      }
    }
  }

  // Join the key slots: each slot summed its own keys (chunk lanes of one slot hold copies of l).
#pragma unroll
  for (int hq = 0; hq < G; ++hq) {
    const float l_tot = slots_sum<CH>(l_run[hq]);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hq][e] = slots_sum<CH>(o[hq][e]);
    if (ks == 0) {
      float* rec = ws + (((size_t)b * H + hk * G + hq) * n_split + split) * REC;
      if (dc == 0) {
        rec[0] = m_run[hq];
        rec[1] = l_tot;
      }
      f32x4* dst = reinterpret_cast<f32x4*>(rec + 4 + dc * 8);
      dst[0] = f32x4{o[hq][0], o[hq][1], o[hq][2], o[hq][3]};
      dst[1] = f32x4{o[hq][4], o[hq][5], o[hq][6], o[hq][7]};
    }
  }
}

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
  const int len = clamp_len(kv_len, b, N_cap);
  const int ns = (len + kDecodeSplit - 1) / kDecodeSplit;
  bf16* out = Od + ((size_t)b * H + h) * HD;
  if (ns == 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) out[lane * PER + e] = to_bf16(0.f);
    if (lse != nullptr && lane == 0) lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  const float* recs = ws + ((size_t)b * H + h) * n_split * REC;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, recs[(size_t)s * REC]);
  float L = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* r = recs + (size_t)s * REC;
    const float wgt = fast_exp2(r[0] - M);
    L = fmaf(wgt, r[1], L);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(wgt, r[4 + lane * PER + e], acc[e]);
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[lane * PER + e] = to_bf16(acc[e] * inv);
  if (lse != nullptr && lane == 0) lse[(size_t)b * H + h] = (M + log2f(L)) * kLn2;
}

template <int HD, int G>
hipError_t launch(const void* q, const void* kc, const void* vc, void* o, float* lse, const int32_t* kv_len,
                  int B, int H, int H_kv, int N_cap, float scale, void* ws, hipStream_t stream,
                  const char* split_name, const char* combine_name) {
  const int n_split = (N_cap + kDecodeSplit - 1) / kDecodeSplit;
  {
    TimedScope ts(split_name, stream);
    hipLaunchKernelGGL((decode_split_kernel<HD, G>), dim3(n_split, H_kv, B), dim3(64), 0, stream,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(kc), static_cast<const bf16*>(vc),
                       kv_len, static_cast<float*>(ws), H, H_kv, N_cap, n_split, scale * kLog2e);
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

template <int HD>
hipError_t launch_g(int G, const void* q, const void* kc, const void* vc, void* o, float* lse,
                    const int32_t* kv_len, int B, int H, int H_kv, int N_cap, float scale, void* ws,
                    hipStream_t stream) {
  switch (G) {
    case 1: return launch<HD, 1>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                 "decode_split_g1", "decode_combine");
    case 2: return launch<HD, 2>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                 "decode_split_g2", "decode_combine");
    case 4: return launch<HD, 4>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                 "decode_split_g4", "decode_combine");
    case 8: return launch<HD, 8>(q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream,
                                 "decode_split_g8", "decode_combine");
    default: return hipErrorInvalidValue;
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
  return d == 128 ? launch_g<128>(G, q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream)
                  : launch_g<64>(G, q, kc, vc, o, lse, kv_len, B, H, H_kv, N_cap, scale, ws, stream);
}

}  // namespace ra
