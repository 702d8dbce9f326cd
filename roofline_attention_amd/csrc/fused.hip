// Forward and backward of attention in one launch on gfx950, with no atomic accumulation.
//
// The MoA paper ("Validating Memory-Optimal Transformer Kernels on Real Hardware", sections
// 4.4-4.5) measures a fused forward+backward that first lost to the unfused pair on the GPU
// because dK and dV were accumulated with atomics, and won once the kernel was restructured so
// that every gradient element has one owner. This kernel keeps that property inside a single
// launch:
//
//   phase 1, one item per pair of query tiles (the causal pairing of the forward): the forward of
//            the tiles (O, LSE), whose epilogue also writes the backward's per-row inputs
//            D_i = sum_c dO[i,c] O[i,c] (stored negated) and LSE_i log2 e; then, in the same workgroup, dQ of the
//            same rows (it needs only those rows' LSE and D, just written by this workgroup);
//   grid barrier (cooperative launch: every workgroup of the grid is resident at once);
//   phase 2, one item per 128-key tile, heaviest (earliest under a causal mask) first, taken from
//            a counter: dK and dV of the tile, streaming Q, dO, LSE, D of every query row (and of
//            every query head of a grouped KV head) that attends to it.
//
// Each item is the same device code as the separate kernels (fwd_bf16_job, bwd_dq_job,
// bwd_dkdv_job), so results match them; D here is summed from the rounded O in a different
// order than in the separate dQ kernel, a float32 rounding-level difference. The one launch takes
// the largest register and LDS footprint of its phases (the key-major item: about 400 registers and
// 97.5 KB of LDS), so every phase runs at one workgroup of 4 waves per CU.
#include <hip/hip_cooperative_groups.h>

#include "bwd_job.hpp"
#include "fwd_bf16_job.hpp"
#include "kernels.hpp"

namespace ra {
namespace {

template <int HD>
constexpr size_t fused_smem_bytes() {
  const size_t a = sizeof(FwdSmem<HD>), b = sizeof(DkdvSmem<HD>), c = sizeof(DqSmem<HD>);
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

static_assert(FWD_THREADS == BWD_THREADS, "the fused kernel runs the forward job with the backward's workgroup");

template <int HD, bool CAUSAL>
__global__ __launch_bounds__(BWD_THREADS, 1) void fwdbwd_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ dQ,
    float* __restrict__ dK, float* __restrict__ dV, float* __restrict__ Dg, float* __restrict__ L2,
    int* __restrict__ counter, int H, int group, int N, int n_t, float scale, float scale_log2, int n_row_items,
    int n_col_items, int n_bhk) {
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  __shared__ int s_item;

  // Phase 1. Items go round-robin over the grid; within a round, consecutive items (query tiles of
  // one head, which share K and V) land on one XCD.
  const int slot = xcd_remap(blockIdx.x, gridDim.x);
  for (int item = slot; item < n_row_items; item += gridDim.x) {
    fwd_bf16_job<HD, CAUSAL, false, true>(Q, K, V, O, LSE, nullptr, 0, H, group, N, n_t, scale_log2,
                                          reinterpret_cast<FwdSmem<HD>*>(dyn_smem), item, dO, Dg, L2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // this item's LSE and D rows are visible to the whole workgroup; LDS is free
    bwd_dq_job<HD, CAUSAL>(Q, K, V, dO, LSE, Dg, dQ, H, group, N, n_t, scale, scale_log2,
                           *reinterpret_cast<DqSmem<HD>*>(dyn_smem), item);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *counter = 0;  // read only after the grid barrier

  cooperative_groups::this_grid().sync();  // every LSE and D row of the batch is written

  // Phase 2. The counter hands out key tiles in order j = kt * n_bhk + bhk: under a causal mask the
  // earliest key tiles carry the most queries, so the longest items start first.
  for (;;) {
    if (threadIdx.x == 0) s_item = atomicAdd(counter, 1);
    __syncthreads();
    const int j = s_item;
    __syncthreads();  // every wave has read s_item before thread 0 takes the next one
    if (j >= n_col_items) break;
    const int item = (j % n_bhk) * n_t + j / n_bhk;  // the key-major item numbering: bhk * n_t + kt
    bwd_dkdv_job<HD, CAUSAL, false, false, false>(Q, K, V, dO, L2, Dg, dK, dV, H, group, N, n_t, scale, scale_log2,
                             *reinterpret_cast<DkdvSmem<HD>*>(dyn_smem), item);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // LDS stages free for the next item
  }
}

template <int HD, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, const void* dout, void* o, float* lse, float* dq,
                  float* dk, float* dv, int B, int H, int H_kv, int N, float scale, void* ws, hipStream_t stream,
                  const char* name) {
  const int n_t = (N + 127) / 128;
  const int n_row_items = (CAUSAL ? (n_t + 1) / 2 : n_t) * H * B;
  const int n_bhk = H_kv * B;
  const int n_col_items = n_t * n_bhk;
  const size_t rows = (size_t)B * H * N;
  float* D = static_cast<float*>(ws);
  float* L2 = D + rows;
  int* counter = reinterpret_cast<int*>(L2 + rows);
  const size_t smem = fused_smem_bytes<HD>();
  auto kernel = &fwdbwd_kernel<HD, CAUSAL>;
  static std::atomic<uint64_t> lds_opt_in{0};  // devices this instantiation's limit is raised on
  hipError_t err = allow_dynamic_lds(lds_opt_in, reinterpret_cast<const void*>(kernel), (int)smem);
  if (err != hipSuccess) return err;
  int dev = 0, per_cu = 0, cus = 0;
  err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess)
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel), BWD_THREADS,
                                                       smem);
  if (err != hipSuccess) return err;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  // Every workgroup of a cooperative grid must be resident; more than the larger phase needs
  // would only wait at the barrier.
  const int need = n_row_items > n_col_items ? n_row_items : n_col_items;
  const int grid = need < per_cu * cus ? need : per_cu * cus;
  const bf16* Q = static_cast<const bf16*>(q);
  const bf16* K = static_cast<const bf16*>(k);
  const bf16* V = static_cast<const bf16*>(v);
  const bf16* dO = static_cast<const bf16*>(dout);
  bf16* O = static_cast<bf16*>(o);
  int group = H / H_kv;
  float scale_log2 = scale * kLog2e;
  void* args[] = {(void*)&Q,     (void*)&K,     (void*)&V,          (void*)&dO,          (void*)&O,
                  (void*)&lse,   (void*)&dq,    (void*)&dk,         (void*)&dv,          (void*)&D,
                  (void*)&L2,    (void*)&counter, (void*)&H,        (void*)&group,       (void*)&N,
                  (void*)&n_t,   (void*)&scale, (void*)&scale_log2, (void*)&n_row_items, (void*)&n_col_items,
                  (void*)&n_bhk};
  TimedScope ts(name, stream);
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid), dim3(BWD_THREADS),
                                    args, (unsigned)smem, stream);
}

}  // namespace

size_t fwdbwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  return 2 * (size_t)B * H * N * sizeof(float) + 16;  // D, LSE * log2 e per query row; the item counter
}

hipError_t launch_fwd_bwd(const void* q, const void* k, const void* v, const void* dout, void* o, float* lse,
                          float* dq, float* dk, float* dv, int B, int H, int H_kv, int N, int d, bool causal,
                          float scale, void* ws, hipStream_t stream) {
  if (d == 128) {
    return causal ? launch<128, true>(q, k, v, dout, o, lse, dq, dk, dv, B, H, H_kv, N, scale, ws, stream,
                                      "fwdbwd_fused_d128_causal")
                  : launch<128, false>(q, k, v, dout, o, lse, dq, dk, dv, B, H, H_kv, N, scale, ws, stream,
                                       "fwdbwd_fused_d128");
  }
  return causal ? launch<64, true>(q, k, v, dout, o, lse, dq, dk, dv, B, H, H_kv, N, scale, ws, stream,
                                   "fwdbwd_fused_d64_causal")
                : launch<64, false>(q, k, v, dout, o, lse, dq, dk, dv, B, H, H_kv, N, scale, ws, stream,
                                    "fwdbwd_fused_d64");
}

}  // namespace ra
