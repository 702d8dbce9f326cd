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
// Kernels, per (batch, head), in this order:
//   bwd_dq  : workgroup = 128 queries (4 waves x 32, Q and dO of its rows in registers); first the
//             rows' D_i = sum_t dO[i,t] O[i,t] (equals sum_j P_ij dP_ij) and LSE_i log2 e, written
//             out (D negated) for the key-major kernel; then it streams 64-key tiles of K and V: S^T = K Q^T,
//             P^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T; stores dQ * scale.
//   bwd_dkdv: workgroup = 128 keys (4 waves x 32, K and V of its keys in registers); streams
//             64-query tiles of Q, dO, LSE and D through three LDS stages:
//             S = Q K^T, P = 2^(S*scale*log2e - LSE*log2e), dV += P^T dO, dP = dO V^T,
//             dS = P (dP - D), dK += dS^T Q; stores dK * scale and dV. Its dP accumulators start
//             at the stored -D, so dS takes one multiply per element.
// MFMA v_mfma_f32_32x32x16_bf16 with fp32 accumulation; P and dS are rounded to bf16 (nearest
// even) as MFMA operands. The probabilities and dS come out of the score accumulators already in
// the A/B-operand layout their next product needs. Operands that contract over the rows of a
// staged tile (dO and Q for dV and dK, K for dQ) come from ds_read_b64_tr_b16 on the row-major
// tile, so nothing is transposed in memory. Tiles reach LDS by direct buffer loads whose range
// check zero-fills rows past the sequence end; zero Q/dO rows and zero K/V rows contribute
// nothing to any stored gradient, so only the causal diagonal needs a mask.
#include "bwd_job.hpp"
#include "kernels.hpp"

namespace ra {
namespace {

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(BWD_THREADS, dkdv_waves_per_simd<HD>()) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dg,
    float* __restrict__ dK, float* __restrict__ dV, int H, int group, int N, int n_ktiles, float scale,
    float scale_log2) {
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  bwd_dkdv_job<HD, CAUSAL>(Q, K, V, dO, LSE2, Dg, dK, dV, H, group, N, n_ktiles, scale, scale_log2,
                           *reinterpret_cast<DkdvSmem<HD>*>(dyn_smem), xcd_remap(blockIdx.x, gridDim.x));
}

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(BWD_THREADS, RA_DQ_WAVES_PER_SIMD) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ O, const bf16* __restrict__ dO, const float* __restrict__ LSE, float* __restrict__ Dg,
    float* __restrict__ L2, float* __restrict__ dQ, int H, int group, int N, int n_qtiles, float scale,
    float scale_log2) {
  __shared__ DqSmem<HD> sm;
  bwd_dq_job<HD, CAUSAL, true>(Q, K, V, dO, LSE, Dg, dQ, H, group, N, n_qtiles, scale, scale_log2, sm,
                               xcd_remap(blockIdx.x, gridDim.x), O, L2);
}

// Ragged batches: the same jobs over packed token rows. The (sequence, head) groups of work items
// are dealt round-robin over the XCDs, as in the ragged forward, so that every XCD gets an equal
// share of every sequence.
template <int HD, bool CAUSAL>
__global__ __launch_bounds__(BWD_THREADS, dkdv_waves_per_simd<HD>()) void bwd_dkdv_varlen_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ Dg,
    float* __restrict__ dK, float* __restrict__ dV, const int32_t* __restrict__ cu_seqlens, int T, int H,
    int group, int N, int n_ktiles, float scale, float scale_log2) {
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  bwd_dkdv_job<HD, CAUSAL, true>(Q, K, V, dO, LSE2, Dg, dK, dV, H, group, N, n_ktiles, scale, scale_log2,
                                 *reinterpret_cast<DkdvSmem<HD>*>(dyn_smem),
                                 xcd_group_remap(blockIdx.x, gridDim.x, n_ktiles), cu_seqlens, T);
}

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(BWD_THREADS, RA_DQ_WAVES_PER_SIMD) void bwd_dq_varlen_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ O, const bf16* __restrict__ dO, const float* __restrict__ LSE, float* __restrict__ Dg,
    float* __restrict__ L2, float* __restrict__ dQ, const int32_t* __restrict__ cu_seqlens, int T, int H,
    int group, int N, int n_qtiles, float scale, float scale_log2) {
  __shared__ DqSmem<HD> sm;
  const int per = CAUSAL ? (n_qtiles + 1) / 2 : n_qtiles;
  bwd_dq_job<HD, CAUSAL, true, true>(Q, K, V, dO, LSE, Dg, dQ, H, group, N, n_qtiles, scale, scale_log2, sm,
                                     xcd_group_remap(blockIdx.x, gridDim.x, group * per), O, L2, cu_seqlens, T);
}

template <int HD, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, float* dq, float* dk, float* dv, int B, int H, int H_kv, int N,
                  float scale, void* ws, hipStream_t stream, const char* dkdv_name, const char* dq_name) {
  const bf16* Q = static_cast<const bf16*>(q);
  const bf16* K = static_cast<const bf16*>(k);
  const bf16* V = static_cast<const bf16*>(v);
  const bf16* O = static_cast<const bf16*>(o);
  const bf16* dO = static_cast<const bf16*>(dout);
  const long long rows = (long long)B * H * N;
  float* D = static_cast<float*>(ws);  // workspace: -D [B,H,N], then LSE * log2 e [B,H,N]
  float* L2 = D + rows;
  const int n_t = (N + 127) / 128;
  const int n_wg = CAUSAL ? (n_t + 1) / 2 : n_t;  // causal workgroups take a pair of tiles
  const int n_wg_kv = CAUSAL && RA_DKDV_PAIR ? (n_t + 1) / 2 : n_t;
  const unsigned total = (unsigned)((long long)n_wg * H * B);           // dQ: per query head
  const unsigned total_kv = (unsigned)((long long)n_wg_kv * H_kv * B);  // dK, dV: per KV head
  // dQ first: it also writes every row's D and LSE * log2 e, which the key-major kernel streams.
  {
    TimedScope ts(dq_name, stream);
    hipLaunchKernelGGL((bwd_dq_kernel<HD, CAUSAL>), dim3(total), dim3(BWD_THREADS), 0, stream, Q, K, V, O, dO, lse,
                       D, L2, dq, H, H / H_kv, N, n_t, scale, scale * kLog2e);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t dkdv_smem = sizeof(DkdvSmem<HD>);
  static std::atomic<uint64_t> lds_opt_in{0};  // devices this instantiation's limit is raised on
  err = allow_dynamic_lds(lds_opt_in, reinterpret_cast<const void*>(&bwd_dkdv_kernel<HD, CAUSAL>), (int)dkdv_smem);
  if (err != hipSuccess) return err;
  {
    TimedScope ts(dkdv_name, stream);
    hipLaunchKernelGGL((bwd_dkdv_kernel<HD, CAUSAL>), dim3(total_kv), dim3(BWD_THREADS), dkdv_smem, stream, Q, K,
                       V, dO, L2, D, dk, dv, H, H / H_kv, N, n_t, scale, scale * kLog2e);
  }
  return hipGetLastError();
}

template <int HD, bool CAUSAL>
hipError_t launch_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, float* dq, float* dk, float* dv, const int32_t* cu_seqlens, int B,
                         int max_seqlen, int T, int H, int H_kv, float scale, void* ws, hipStream_t stream,
                         const char* dkdv_name, const char* dq_name) {
  const bf16* Q = static_cast<const bf16*>(q);
  const bf16* K = static_cast<const bf16*>(k);
  const bf16* V = static_cast<const bf16*>(v);
  const bf16* O = static_cast<const bf16*>(o);
  const bf16* dO = static_cast<const bf16*>(dout);
  float* D = static_cast<float*>(ws);  // workspace: -D [H,T], then LSE * log2 e [H,T]
  float* L2 = D + (size_t)H * T;
  const int n_t = (max_seqlen + 127) / 128;
  const int n_wg = CAUSAL ? (n_t + 1) / 2 : n_t;
  const unsigned total = (unsigned)((long long)n_wg * H * B);
  const unsigned total_kv = (unsigned)((long long)n_t * H_kv * B);
  {
    TimedScope ts(dq_name, stream);
    hipLaunchKernelGGL((bwd_dq_varlen_kernel<HD, CAUSAL>), dim3(total), dim3(BWD_THREADS), 0, stream, Q, K, V, O,
                       dO, lse, D, L2, dq, cu_seqlens, T, H, H / H_kv, max_seqlen, n_t, scale, scale * kLog2e);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t dkdv_smem = sizeof(DkdvSmem<HD>);
  static std::atomic<uint64_t> lds_opt_in{0};  // devices this instantiation's limit is raised on
  err = allow_dynamic_lds(lds_opt_in, reinterpret_cast<const void*>(&bwd_dkdv_varlen_kernel<HD, CAUSAL>), (int)dkdv_smem);
  if (err != hipSuccess) return err;
  {
    TimedScope ts(dkdv_name, stream);
    hipLaunchKernelGGL((bwd_dkdv_varlen_kernel<HD, CAUSAL>), dim3(total_kv), dim3(BWD_THREADS), dkdv_smem, stream,
                       Q, K, V, dO, L2, D, dk, dv, cu_seqlens, T, H, H / H_kv, max_seqlen, n_t, scale,
                       scale * kLog2e);
  }
  return hipGetLastError();
}

}  // namespace

size_t bwd_varlen_workspace_bytes(int T, int H, int d) {
  (void)d;
  return 2 * (size_t)H * T * sizeof(float);  // -D and LSE * log2 e per (head, token) row
}

hipError_t launch_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, float* dq, float* dk, float* dv, const int32_t* cu_seqlens, int B,
                             int max_seqlen, int T, int H, int H_kv, int d, bool causal, float scale, void* ws,
                             hipStream_t stream) {
  if (d == 128) {
    return causal ? launch_varlen<128, true>(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, max_seqlen, T, H, H_kv,
                                             scale, ws, stream, "bwd_dkdv_varlen_d128_causal",
                                             "bwd_dq_varlen_d128_causal")
                  : launch_varlen<128, false>(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, max_seqlen, T, H,
                                              H_kv, scale, ws, stream, "bwd_dkdv_varlen_d128", "bwd_dq_varlen_d128");
  }
  return causal ? launch_varlen<64, true>(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, max_seqlen, T, H, H_kv,
                                          scale, ws, stream, "bwd_dkdv_varlen_d64_causal", "bwd_dq_varlen_d64_causal")
                : launch_varlen<64, false>(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, max_seqlen, T, H, H_kv,
                                           scale, ws, stream, "bwd_dkdv_varlen_d64", "bwd_dq_varlen_d64");
}

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  return 2 * (size_t)B * H * N * sizeof(float);  // -D and LSE * log2 e per query row
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* dq, float* dk, float* dv, int B, int H, int H_kv, int N, int d,
                      bool causal, float scale, void* ws, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch<128, true>(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, scale, ws, stream,
                                      "bwd_dkdv_d128_causal", "bwd_dq_d128_causal")
                  : launch<128, false>(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, scale, ws, stream,
                                       "bwd_dkdv_d128", "bwd_dq_d128");
  }
  return causal ? launch<64, true>(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, scale, ws, stream,
                                   "bwd_dkdv_d64_causal", "bwd_dq_d64_causal")
                : launch<64, false>(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, scale, ws, stream,
                                    "bwd_dkdv_d64", "bwd_dq_d64");
}

}  // namespace ra
