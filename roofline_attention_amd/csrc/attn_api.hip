// C-ABI layer of libroofattn.so: argument validation, dispatch to the kernel launchers, status
// strings and the opt-in kernel timer. Every check runs before any HIP call, so a rejected call
// has no side effects on the device.
#include <float.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "kernels.hpp"

namespace {

thread_local std::string t_last_error;

attn_status fail(attn_status st, const char* msg) {
  t_last_error = msg;
  return st;
}

attn_status ok() {
  t_last_error.clear();
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t bytes;
};

bool overlap(Range a, Range b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Common shape checks; returns ATTN_OK or the failing status (message already set).
attn_status check_shape(int B, int H, int H_kv, int N, int d, float scale) {
  if (B < 1 || H < 1 || H_kv < 1 || N < 1) return fail(ATTN_ERR_INVALID_ARG, "B, H, H_kv and N must be >= 1");
  if (H % H_kv != 0) return fail(ATTN_ERR_INVALID_ARG, "H must be a multiple of H_kv");
  if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "head dimension d must be 64 or 128");
  if ((long long)N * d > (1LL << 30)) return fail(ATTN_ERR_INVALID_ARG, "N * d exceeds 2^30");
  if (B > 65535 || H > 65535) return fail(ATTN_ERR_INVALID_ARG, "B and H must be <= 65535");
  if (!isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "scale must be finite");
  return ATTN_OK;
}

attn_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  t_last_error = std::string("HIP launch error: ") + hipGetErrorString(e);
  return ATTN_ERR_HIP;
}

// ---------------------------------------------------------------------------- timer ----

struct TimerRecord {
  std::string name;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  long long launches = 0;
  double total_ms = 0.0;
  std::vector<float> samples;  // duration of every drained launch, in launch order (ms)
};

std::mutex g_mu;
bool g_timing = false;
std::vector<TimerRecord> g_records;
std::vector<hipEvent_t> g_free_events;

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

TimerRecord& record_for(const char* name) {
  for (auto& r : g_records)
    if (r.name == name) return r;
  g_records.push_back(TimerRecord{});
  g_records.back().name = name;
  return g_records.back();
}

attn_status drain_locked() {
  for (auto& r : g_records) {
    for (auto& pr : r.pending) {
      if (hipEventSynchronize(pr.second) != hipSuccess) return fail(ATTN_ERR_HIP, "event synchronize failed");
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
        return fail(ATTN_ERR_HIP, "event elapsed time failed");
      r.total_ms += ms;
      r.launches += 1;
      r.samples.push_back(ms);
      g_free_events.push_back(pr.first);
      g_free_events.push_back(pr.second);
    }
    r.pending.clear();
  }
  return ATTN_OK;
}

}  // namespace

namespace ra {

TimedScope::TimedScope(const char* name, hipStream_t stream) : name_(name), stream_(stream), start_(nullptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_timing) return;
  hipEvent_t e = take_event();
  if (e != nullptr && hipEventRecord(e, stream_) == hipSuccess) start_ = e;
}

TimedScope::~TimedScope() {
  if (start_ == nullptr) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = take_event();
  if (e == nullptr || hipEventRecord(e, stream_) != hipSuccess) return;
  record_for(name_).pending.emplace_back(static_cast<hipEvent_t>(start_), e);
}

}  // namespace ra

extern "C" {

int attn_abi_version(void) { return 7; }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
    default: return "ATTN_ERR_UNKNOWN";
  }
}

const char* attn_last_error(void) { return t_last_error.c_str(); }

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                     int N, int d, int causal, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  attn_status st = check_shape(B, H, H_kv, N, d, scale);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "dtype must be ATTN_F32 or ATTN_BF16");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t es = dtype == ATTN_F32 ? 4 : 2;
  const size_t qb = (size_t)B * H * N * d * es, kb = (size_t)B * H_kv * N * d * es, lb = (size_t)B * H * N * 4;
  const Range rq{q, qb}, rk{k, kb}, rv{v, kb}, ro{o, qb}, rl{lse, lse ? lb : 0};
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) || overlap(rl, rk) ||
      overlap(rl, rv) || overlap(rl, ro))
    return fail(ATTN_ERR_INVALID_ARG, "outputs overlap inputs or each other");
  const long long tiles = (long long)((N + 63) / 64) * H * B;
  if (tiles > 0x7fffffffLL) return fail(ATTN_ERR_INVALID_ARG, "problem too large for one launch");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_F32)
    return hip_status(ra::launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                         static_cast<const float*>(v), static_cast<float*>(o), lse, B, H, H_kv, N, d,
                                         causal != 0, scale, s));
  return hip_status(ra::launch_fwd_bf16(q, k, v, o, lse, B, H, H_kv, N, d, causal != 0, scale, s));
}

attn_status attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                         int N, int d, int causal, float scale, float q_descale, float k_descale, float v_descale,
                         void* stream) {
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  attn_status st = check_shape(B, H, H_kv, N, d, scale);
  if (st != ATTN_OK) return st;
  if (!isfinite(q_descale) || !isfinite(k_descale) || !isfinite(v_descale))
    return fail(ATTN_ERR_INVALID_ARG, "descale factors must be finite");
  if (!(fabs((double)scale * q_descale * k_descale * 1.4426950408889634) <= (double)FLT_MAX))
    return fail(ATTN_ERR_INVALID_ARG, "scale * q_descale * k_descale overflows float32");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t qb = (size_t)B * H * N * d, kb = (size_t)B * H_kv * N * d, ob = qb * 2, lb = (size_t)B * H * N * 4;
  const Range rq{q, qb}, rk{k, kb}, rv{v, kb}, ro{o, ob}, rl{lse, lse ? lb : 0};
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(rl, rq) || overlap(rl, rk) ||
      overlap(rl, rv) || overlap(rl, ro))
    return fail(ATTN_ERR_INVALID_ARG, "outputs overlap inputs or each other");
  const long long tiles = (long long)((N + 127) / 128) * H * B;
  if (tiles > 0x7fffffffLL) return fail(ATTN_ERR_INVALID_ARG, "problem too large for one launch");
  return hip_status(ra::launch_fwd_fp8(q, k, v, o, lse, B, H, H_kv, N, d, causal != 0, scale, q_descale, k_descale,
                                       v_descale, static_cast<hipStream_t>(stream)));
}

attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens, int B, int max_seqlen, int T, int H, int H_kv, int d,
                            int causal, float scale, int dtype, void* stream) {
  if (!q || !k || !v || !o || !cu_seqlens)
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v, o and cu_seqlens must be non-null");
  if (T < 0) return fail(ATTN_ERR_INVALID_ARG, "T must be >= 0");
  attn_status st = check_shape(B, H, H_kv, max_seqlen, d, scale);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "ragged prefill supports ATTN_BF16 only");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "cu_seqlens and lse must be 4-byte aligned");
  const size_t qb = (size_t)T * H * d * 2, kb = (size_t)T * H_kv * d * 2, lb = (size_t)H * T * 4;
  const Range rq{q, qb}, rk{k, kb}, rv{v, kb}, ro{o, qb}, rl{lse, lse ? lb : 0}, rc{cu_seqlens, (size_t)(B + 1) * 4};
  const Range outs[] = {ro, rl};
  const Range ins[] = {rq, rk, rv, rc};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ATTN_ERR_INVALID_ARG, "outputs overlap inputs");
  if (overlap(ro, rl)) return fail(ATTN_ERR_INVALID_ARG, "o and lse overlap");
  const long long tiles = (long long)((max_seqlen + 63) / 64) * H * B;
  if (tiles > 0x7fffffffLL) return fail(ATTN_ERR_INVALID_ARG, "problem too large for one launch");
  if (T == 0) return ok();  // no rows
  return hip_status(ra::launch_fwd_bf16_varlen(q, k, v, o, lse, cu_seqlens, B, max_seqlen, T, H, H_kv, d,
                                               causal != 0, scale, static_cast<hipStream_t>(stream)));
}

size_t attn_decode_workspace_size(int B, int H, int N_cap, int d) {
  if (B < 1 || H < 1 || N_cap < 1 || (d != 64 && d != 128)) return 0;
  return ra::decode_workspace_bytes(B, H, N_cap, d);
}

}  // extern "C"

namespace {

// Checks of a contiguous decode call shared by attn_decode and attn_decode_noalloc; `workspace`
// (need bytes) is the caller's buffer, or nullptr for the library's fixed scratch, which cannot
// overlap caller memory.
attn_status check_decode(const void* q, const void* k_cache, const void* v_cache, const void* o, const float* lse,
                         const int32_t* kv_len, int B, int H, int H_kv, int N_cap, int d, float scale, int dtype,
                         const void* workspace, size_t need) {
  if (!q || !k_cache || !v_cache || !o || !kv_len)
    return fail(ATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, o and kv_len must be non-null");
  attn_status st = check_shape(B, H, H_kv, N_cap, d, scale);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "decode supports ATTN_BF16 only");
  const int G = H / H_kv;
  const long long chunks = (G == 1 || G == 2 || G == 4 || G == 8) ? 1 : (G + 15) / 16;
  if ((long long)B * H_kv * chunks >= (1LL << 24))
    return fail(ATTN_ERR_INVALID_ARG, "decode needs B * H_kv * ceil(G / 16) < 2^24 (one grid row of workgroups)");
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, caches and o must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(kv_len) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "kv_len and lse must be 4-byte aligned");
  const size_t qb = (size_t)B * H * d * 2, cb = (size_t)B * H_kv * N_cap * d * 2;
  const Range rq{q, qb}, rk{k_cache, cb}, rv{v_cache, cb}, ro{o, qb}, rl{lse, lse ? (size_t)B * H * 4 : 0},
      rw{workspace, workspace ? need : 0}, rn{kv_len, (size_t)B * 4};
  const Range outs[] = {ro, rl, rw};
  const Range ins[] = {rq, rk, rv, rn};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap inputs");
  if (overlap(ro, rl) || overlap(ro, rw) || overlap(rl, rw))
    return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap each other");
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                        const int32_t* kv_len, int B, int H, int H_kv, int N_cap, int d, int causal, float scale,
                        int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  (void)causal;
  attn_status st = check_decode(q, k_cache, v_cache, o, lse, kv_len, B, H, H_kv, N_cap, d, scale, dtype, nullptr, 0);
  if (st != ATTN_OK) return st;
  const size_t need = ra::decode_workspace_bytes(B, H, N_cap, d);
  if (workspace == nullptr || workspace_bytes < need) return fail(ATTN_ERR_WORKSPACE, "decode workspace too small");
  if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  st = check_decode(q, k_cache, v_cache, o, lse, kv_len, B, H, H_kv, N_cap, d, scale, dtype, workspace, need);
  if (st != ATTN_OK) return st;
  return hip_status(ra::launch_decode(q, k_cache, v_cache, o, lse, kv_len, B, H, H_kv, N_cap, d, scale, workspace,
                                      static_cast<hipStream_t>(stream)));
}

attn_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                const int32_t* kv_len, int B, int H, int H_kv, int N_cap, int d, int causal,
                                float scale, int dtype, void* stream) {
  (void)causal;
  attn_status st = check_decode(q, k_cache, v_cache, o, lse, kv_len, B, H, H_kv, N_cap, d, scale, dtype, nullptr, 0);
  if (st != ATTN_OK) return st;
  const size_t need = ra::decode_workspace_bytes(B, H, N_cap, d);
  if (need > ATTN_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(ATTN_ERR_WORKSPACE,
                "attn_decode_noalloc: B * H * ceil(N_cap / 1024) * (d + 4) * 4 bytes of split records exceed the "
                "library's fixed scratch (ATTN_DECODE_NOALLOC_SCRATCH_BYTES); use attn_decode with a workspace");
  void* scratch = nullptr;
  const hipError_t e = ra::decode_scratch_address(&scratch);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(ra::launch_decode(q, k_cache, v_cache, o, lse, kv_len, B, H, H_kv, N_cap, d, scale, scratch,
                                      static_cast<hipStream_t>(stream)));
}

attn_status attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse,
                              const int32_t* kv_len, const int32_t* block_table, int B, int H, int H_kv,
                              int num_pages, int page_size, int max_pages, int d, float scale, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_pages || !v_pages || !o || !kv_len || !block_table)
    return fail(ATTN_ERR_INVALID_ARG, "q, k_pages, v_pages, o, kv_len and block_table must be non-null");
  if (page_size < 32 || page_size > 1024 || (page_size & (page_size - 1)))
    return fail(ATTN_ERR_UNSUPPORTED, "page_size must be a power of two in [32, 1024]");
  if (num_pages < 1 || max_pages < 1) return fail(ATTN_ERR_INVALID_ARG, "num_pages and max_pages must be >= 1");
  const long long n_cap = (long long)max_pages * page_size;
  if (n_cap > 0x7fffffffLL) return fail(ATTN_ERR_INVALID_ARG, "max_pages * page_size exceeds 2^31 - 1");
  const int N_cap = (int)n_cap;
  attn_status st = check_shape(B, H, H_kv, N_cap, d, scale);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "decode supports ATTN_BF16 only");
  const int G = H / H_kv;
  const long long chunks = (G == 1 || G == 2 || G == 4 || G == 8) ? 1 : (G + 15) / 16;
  if ((long long)B * H_kv * chunks >= (1LL << 24))
    return fail(ATTN_ERR_INVALID_ARG, "decode needs B * H_kv * ceil(G / 16) < 2^24 (one grid row of workgroups)");
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "q, pages and o must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(kv_len) & 3u) || (reinterpret_cast<uintptr_t>(block_table) & 3u) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(ATTN_ERR_INVALID_ARG, "kv_len, block_table and lse must be 4-byte aligned");
  const size_t need = ra::decode_workspace_bytes(B, H, N_cap, d);
  if (workspace == nullptr || workspace_bytes < need) return fail(ATTN_ERR_WORKSPACE, "decode workspace too small");
  if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const size_t qb = (size_t)B * H * d * 2, pb = (size_t)num_pages * H_kv * page_size * d * 2;
  const Range rq{q, qb}, rk{k_pages, pb}, rv{v_pages, pb}, ro{o, qb}, rl{lse, lse ? (size_t)B * H * 4 : 0},
      rw{workspace, need}, rn{kv_len, (size_t)B * 4}, rt{block_table, (size_t)B * max_pages * 4};
  const Range outs[] = {ro, rl, rw};
  const Range ins[] = {rq, rk, rv, rn, rt};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap inputs");
  if (overlap(ro, rl) || overlap(ro, rw) || overlap(rl, rw))
    return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap each other");
  return hip_status(ra::launch_decode_paged(q, k_pages, v_pages, o, lse, kv_len, block_table, B, H, H_kv, num_pages,
                                            page_size, max_pages, d, scale, workspace,
                                            static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return ra::bwd_workspace_bytes(B, H, N, d);
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     float* dq, float* dk, float* dv, int B, int H, int H_kv, int N, int d, int causal, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(ATTN_ERR_INVALID_ARG, "all tensor pointers must be non-null");
  attn_status st = check_shape(B, H, H_kv, N, d, scale);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "backward supports ATTN_BF16 only");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(ATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t need = ra::bwd_workspace_bytes(B, H, N, d);
  if (workspace == nullptr || workspace_bytes < need) return fail(ATTN_ERR_WORKSPACE, "backward workspace too small");
  if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const long long tiles = (long long)((N + 127) / 128) * H * B;
  if (tiles > 0x7fffffffLL) return fail(ATTN_ERR_INVALID_ARG, "problem too large for one launch");
  const size_t tb = (size_t)B * H * N * d * 2, kb = (size_t)B * H_kv * N * d * 2, gb = (size_t)B * H * N * d * 4,
               gkb = (size_t)B * H_kv * N * d * 4, lb = (size_t)B * H * N * 4;
  const Range ins[] = {{q, tb}, {k, kb}, {v, kb}, {o, tb}, {dout, tb}, {lse, lb}};
  const Range outs[] = {{dq, gb}, {dk, gkb}, {dv, gkb}, {workspace, need}};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap inputs");
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap each other");
  return hip_status(ra::launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, H_kv, N, d, causal != 0, scale, workspace,
                                   static_cast<hipStream_t>(stream)));
}

size_t attn_bwd_varlen_workspace_size(int T, int H, int d) {
  if (T < 0 || H < 1 || (d != 64 && d != 128)) return 0;
  return ra::bwd_varlen_workspace_bytes(T, H, d);
}

attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, float* dq, float* dk, float* dv, const int32_t* cu_seqlens, int B,
                            int max_seqlen, int T, int H, int H_kv, int d, int causal, float scale, int dtype,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !cu_seqlens)
    return fail(ATTN_ERR_INVALID_ARG, "all tensor pointers and cu_seqlens must be non-null");
  if (T < 0) return fail(ATTN_ERR_INVALID_ARG, "T must be >= 0");
  attn_status st = check_shape(B, H, H_kv, max_seqlen, d, scale);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "ragged backward supports ATTN_BF16 only");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(ATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return fail(ATTN_ERR_INVALID_ARG, "lse and cu_seqlens must be 4-byte aligned");
  const size_t need = ra::bwd_varlen_workspace_bytes(T, H, d);
  if (T > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(ATTN_ERR_WORKSPACE, "ragged backward workspace too small");
  if (workspace && !aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const long long tiles = (long long)((max_seqlen + 127) / 128) * H * B;
  if (tiles > 0x7fffffffLL) return fail(ATTN_ERR_INVALID_ARG, "problem too large for one launch");
  const size_t tb = (size_t)T * H * d * 2, kb = (size_t)T * H_kv * d * 2, gb = (size_t)T * H * d * 4,
               gkb = (size_t)T * H_kv * d * 4, lb = (size_t)H * T * 4;
  const Range ins[] = {{q, tb}, {k, kb}, {v, kb}, {o, tb}, {dout, tb}, {lse, lb}, {cu_seqlens, (size_t)(B + 1) * 4}};
  const Range outs[] = {{dq, gb}, {dk, gkb}, {dv, gkb}, {workspace, T > 0 ? need : 0}};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap inputs");
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outs[j])) return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap each other");
  if (T == 0) return ok();  // no rows
  return hip_status(ra::launch_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, B, max_seqlen, T, H, H_kv,
                                          d, causal != 0, scale, workspace, static_cast<hipStream_t>(stream)));
}

size_t attn_fwd_bwd_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  return ra::fwdbwd_workspace_bytes(B, H, N, d);
}

attn_status attn_fwd_bwd(const void* q, const void* k, const void* v, const void* dout, void* o, float* lse,
                         float* dq, float* dk, float* dv, int B, int H, int H_kv, int N, int d, int causal,
                         float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !dout || !o || !lse || !dq || !dk || !dv)
    return fail(ATTN_ERR_INVALID_ARG, "all tensor pointers must be non-null");
  attn_status st = check_shape(B, H, H_kv, N, d, scale);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return fail(ATTN_ERR_UNSUPPORTED, "the fused forward+backward supports ATTN_BF16 only");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return fail(ATTN_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(ATTN_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  const size_t need = ra::fwdbwd_workspace_bytes(B, H, N, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(ATTN_ERR_WORKSPACE, "fused forward+backward workspace too small");
  if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const long long tiles = (long long)((N + 127) / 128) * H * B;
  if (tiles > 0x7fffffffLL) return fail(ATTN_ERR_INVALID_ARG, "problem too large for one launch");
  const size_t tb = (size_t)B * H * N * d * 2, kb = (size_t)B * H_kv * N * d * 2, gb = (size_t)B * H * N * d * 4,
               gkb = (size_t)B * H_kv * N * d * 4, lb = (size_t)B * H * N * 4;
  const Range ins[] = {{q, tb}, {k, kb}, {v, kb}, {dout, tb}};
  const Range outs[] = {{o, tb}, {lse, lb}, {dq, gb}, {dk, gkb}, {dv, gkb}, {workspace, need}};
  for (const Range& a : outs)
    for (const Range& b : ins)
      if (overlap(a, b)) return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap inputs");
  for (int i = 0; i < 6; ++i)
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outs[j])) return fail(ATTN_ERR_INVALID_ARG, "outputs or workspace overlap each other");
  return hip_status(ra::launch_fwd_bwd(q, k, v, dout, o, lse, dq, dk, dv, B, H, H_kv, N, d, causal != 0, scale,
                                       workspace, static_cast<hipStream_t>(stream)));
}

attn_status attn_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_timing = on != 0;
  return ok();
}

attn_status attn_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  attn_status st = drain_locked();
  g_records.clear();
  return st == ATTN_OK ? ok() : st;
}

int attn_timing_samples(int index, float* ms, int cap) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (index < 0 || index >= (int)g_records.size()) {
    fail(ATTN_ERR_INVALID_ARG, "timer index out of range");
    return -1;
  }
  if (cap < 0 || (cap > 0 && ms == nullptr)) {
    fail(ATTN_ERR_INVALID_ARG, "ms must hold cap >= 0 floats");
    return -1;
  }
  if (drain_locked() != ATTN_OK) return -1;
  const std::vector<float>& v = g_records[index].samples;
  const int n = (int)v.size();
  for (int i = 0; i < n && i < cap; ++i) ms[i] = v[i];
  ok();
  return n;
}

attn_status attn_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_timing = false;
  attn_status st = drain_locked();  // waits for every recorded event before it is destroyed
  for (auto& r : g_records)
    for (auto& pr : r.pending) g_free_events.push_back(pr.first), g_free_events.push_back(pr.second);
  g_records.clear();
  bool destroyed = true;
  for (hipEvent_t e : g_free_events) destroyed = hipEventDestroy(e) == hipSuccess && destroyed;
  g_free_events.clear();
  g_free_events.shrink_to_fit();
  if (st != ATTN_OK) return st;
  return destroyed ? ok() : fail(ATTN_ERR_HIP, "hipEventDestroy failed");
}

int attn_timing_count(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return (int)g_records.size();
}

attn_status attn_timing_get(int index, const char** name, long long* launches, double* total_ms) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (index < 0 || index >= (int)g_records.size()) return fail(ATTN_ERR_INVALID_ARG, "timer index out of range");
  attn_status st = drain_locked();
  if (st != ATTN_OK) return st;
  const TimerRecord& r = g_records[index];
  if (name) *name = r.name.c_str();
  if (launches) *launches = r.launches;
  if (total_ms) *total_ms = r.total_ms;
  return ok();
}

}  // extern "C"
