// Fused tiled attention forward for bf16 inputs on gfx950: the kernels and their launchers. The
// work of one workgroup (schedule, tiling, gfx950 mapping) is fwd_bf16_job in fwd_bf16_job.hpp.
#include "fwd_bf16_job.hpp"
#include "kernels.hpp"

namespace ra {
namespace {

template <int HD, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(FWD_THREADS, 8 / FWD_WAVES) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ cu_seqlens, int T, int H,
    int group, int N, int n_qtiles, float scale_log2, int split_pairs) {
  // A ragged batch deals the KV-head groups of its sequences round-robin over the XCDs (sequence
  // lengths differ, so a contiguous split would load the XCDs unevenly); a dense batch keeps
  // consecutive items (one head's tiles) together on an XCD. With split_pairs the grid is twice
  // the pair count: workgroups L and L + half run the heavy and the light tile of one pair.
  const int per_head = CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles;
  if (split_pairs) {
    const int half = gridDim.x / 2;
    fwd_bf16_job<HD, CAUSAL, VARLEN, false>(Q, K, V, O, LSE, cu_seqlens, T, H, group, N, n_qtiles, scale_log2,
                                            nullptr, xcd_remap(blockIdx.x % half, half), nullptr, nullptr,
                                            nullptr, (int)(blockIdx.x / half));
    return;
  }
  const int item = VARLEN ? xcd_group_remap(blockIdx.x, gridDim.x, group * per_head)
                          : xcd_remap(blockIdx.x, gridDim.x);
  fwd_bf16_job<HD, CAUSAL, VARLEN, false>(Q, K, V, O, LSE, cu_seqlens, T, H, group, N, n_qtiles, scale_log2,
                                          nullptr, item, nullptr, nullptr, nullptr);
}

template <int HD, bool CAUSAL, bool VARLEN>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_seqlens, int T,
                  int B, int H, int H_kv, int N, float scale, hipStream_t stream, const char* name) {
  const int n_qt = (N + FWD_BR - 1) / FWD_BR;
  long long total = (long long)(CAUSAL ? (n_qt + 1) / 2 : n_qt) * H * B;
  // A causal grid of pairs that fills fewer than two workgroups per CU runs each pair as two
  // workgroups (measured on [4,16,1024,64]: 335 -> 380 TFLOP/s; on grids that fill the chip the
  // pairs stay together: [2,32,4096,128] 825 vs 787).
  const int cus = device_cus();
  const int split = CAUSAL && !VARLEN && cus > 0 && total < 2LL * cus ? 1 : 0;
  if (split) total *= 2;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  TimedScope ts(name, stream);
  hipLaunchKernelGGL((fwd_bf16_kernel<HD, CAUSAL, VARLEN>), dim3((unsigned)total), dim3(FWD_THREADS), 0, stream,
                     static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                     static_cast<bf16*>(o), lse, cu_seqlens, T, H, H / H_kv, N, n_qt, scale * kLog2e, split);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                           int H, int H_kv, int N, int d, bool causal, float scale, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch<128, true, false>(q, k, v, o, lse, nullptr, 0, B, H, H_kv, N, scale, stream,
                                             "fwd_bf16_d128_causal")
                  : launch<128, false, false>(q, k, v, o, lse, nullptr, 0, B, H, H_kv, N, scale, stream,
                                              "fwd_bf16_d128");
  }
  return causal ? launch<64, true, false>(q, k, v, o, lse, nullptr, 0, B, H, H_kv, N, scale, stream,
                                          "fwd_bf16_d64_causal")
                : launch<64, false, false>(q, k, v, o, lse, nullptr, 0, B, H, H_kv, N, scale, stream, "fwd_bf16_d64");
}

hipError_t launch_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const int32_t* cu_seqlens, int B, int max_seqlen, int T, int H, int H_kv, int d,
                                  bool causal, float scale, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch<128, true, true>(q, k, v, o, lse, cu_seqlens, T, B, H, H_kv, max_seqlen, scale, stream,
                                            "fwd_bf16_varlen_d128_causal")
                  : launch<128, false, true>(q, k, v, o, lse, cu_seqlens, T, B, H, H_kv, max_seqlen, scale, stream,
                                             "fwd_bf16_varlen_d128");
  }
  return causal ? launch<64, true, true>(q, k, v, o, lse, cu_seqlens, T, B, H, H_kv, max_seqlen, scale, stream,
                                         "fwd_bf16_varlen_d64_causal")
                : launch<64, false, true>(q, k, v, o, lse, cu_seqlens, T, B, H, H_kv, max_seqlen, scale, stream,
                                          "fwd_bf16_varlen_d64");
}

}  // namespace ra
