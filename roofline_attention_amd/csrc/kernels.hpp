// Host-side launchers of the attention kernels (internal to libroofattn.so).
// Each launcher assumes its arguments were validated by the C-ABI layer and returns the
// hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace ra {

// Raises a kernel's dynamic-LDS limit to `bytes` once per device (bit d of `done` marks device
// d; the attribute is per device). Safe to call from several host threads: the call is idempotent
// and the mark is atomic.
inline hipError_t allow_dynamic_lds(std::atomic<uint64_t>& done, const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Compute units of the current device, or 0 if the runtime cannot say.
inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

// Brackets one kernel launch with timing events when the opt-in timer is enabled.
class TimedScope {
 public:
  TimedScope(const char* name, hipStream_t stream);
  ~TimedScope();
  TimedScope(const TimedScope&) = delete;
  TimedScope& operator=(const TimedScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  void* start_;
};

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int H_kv, int N, int d, bool causal, float scale,
                           hipStream_t stream);

// Ragged prefill over packed rows: q, o [T,H,d], k, v [T,H_kv,d], lse [H,T]; sequence b is rows
// cu_seqlens[b] .. cu_seqlens[b+1] - 1 (device array), each at most max_seqlen long.
hipError_t launch_fwd_bf16_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                  const int32_t* cu_seqlens, int B, int max_seqlen, int T, int H, int H_kv, int d,
                                  bool causal, float scale, hipStream_t stream);

// fp8 (E4M3) inputs, d = 64 or 128: q [B,H,N,d], k, v [B,H_kv,N,d] uint8 codes; o bf16; real inputs
// are descale * decoded code.
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                          int N, int d, bool causal, float scale, float q_descale, float k_descale, float v_descale,
                          hipStream_t stream);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int B, int H, int H_kv, int N, int d, bool causal, float scale,
                          hipStream_t stream);

// Decode: the least number of keys one split-kernel workgroup streams (its share of the batch's
// keys is at least this long), and the workspace layout: per (b, h) ceil(N_cap / kDecodeSplit) + 1
// record slots of d + 4 floats {m, l, np, -, o[0..d)} (m in log2 units of the scaled score, o not
// yet divided by l, np the segment's record count as int bits), one per workgroup share that meets
// the segment.
#ifndef RA_DECODE_SPLIT
#define RA_DECODE_SPLIT 1024
#endif
constexpr int kDecodeSplit = RA_DECODE_SPLIT;
size_t decode_workspace_bytes(int B, int H, int N_cap, int d);
hipError_t launch_decode(const void* q, const void* kc, const void* vc, void* o, float* lse,
                         const int32_t* kv_len, int B, int H, int H_kv, int N_cap, int d,
                         float scale, void* ws, hipStream_t stream);
// Device address of the library's fixed decode scratch (ATTN_DECODE_NOALLOC_SCRATCH_BYTES) on the
// current device, looked up once per device and cached.
hipError_t decode_scratch_address(void** ptr);

// Paged caches: k_pages, v_pages [num_pages, H_kv, page_size, d], block_table [B, max_pages] of
// physical page ids; page_size a power of two in [32, 1024]. Same workspace as launch_decode with
// N_cap = max_pages * page_size.
hipError_t launch_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse,
                               const int32_t* kv_len, const int32_t* block_table, int B, int H, int H_kv,
                               int num_pages, int page_size, int max_pages, int d, float scale, void* ws,
                               hipStream_t stream);

size_t bwd_workspace_bytes(int B, int H, int N, int d);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, float* dq, float* dk, float* dv,
                      int B, int H, int H_kv, int N, int d, bool causal, float scale, void* ws,
                      hipStream_t stream);
// Ragged backward over packed rows (layouts of launch_fwd_bf16_varlen; lse [H, T]); the
// workspace holds D and LSE * log2 e as [H, T] each.
size_t bwd_varlen_workspace_bytes(int T, int H, int d);
hipError_t launch_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, float* dq, float* dk, float* dv, const int32_t* cu_seqlens, int B,
                             int max_seqlen, int T, int H, int H_kv, int d, bool causal, float scale, void* ws,
                             hipStream_t stream);

// Forward and backward in one cooperative launch: o, lse from the forward and dq, dk, dv from the
// backward, with the workspace holding D, LSE * log2 e and an item counter.
size_t fwdbwd_workspace_bytes(int B, int H, int N, int d);
hipError_t launch_fwd_bwd(const void* q, const void* k, const void* v, const void* dout, void* o, float* lse,
                          float* dq, float* dk, float* dv, int B, int H, int H_kv, int N, int d, bool causal,
                          float scale, void* ws, hipStream_t stream);

}  // namespace ra
