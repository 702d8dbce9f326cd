/*
 * attn.h - C ABI of the MI355X (gfx950) exact-attention library libroofattn.so.
 *
 * Operation: exact scaled-dot-product attention, O = softmax(scale * Q K^T [+ causal mask]) V,
 * as defined in "Why Fast GPUs Still Wait for Memory", section "Attention from first principles"
 * (S = Q K^T, P = softmax(S), O = P V), computed by fused tiled kernels that keep S and P on chip
 * (same page, section "FlashAttention is an IO algorithm"). The score factor `scale` is a free
 * argument (the page writes S = Q K^T without it; callers normally pass 1/sqrt(d)).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers (memory of the current HIP device), 16-byte aligned,
 *     densely packed row-major with the head dimension d contiguous:
 *       Q, O, dO, dQ : [B, H,    N, d]       K, V, dK, dV : [B, H_kv, N, d]
 *       LSE          : [B, H, N] float32, natural-log log-sum-exp of each score row.
 *   - Grouped-query attention: H must be a multiple of H_kv; query head h reads KV head
 *     h / (H / H_kv) (contiguous groups), as in "Why Fast GPUs Still Wait for Memory",
 *     section "Attention III - KV cache, GQA, MLA" (group size g = h / h_kv).
 *   - causal != 0 keeps key j for query i only when j <= i (lower triangle with the diagonal;
 *     same page, note "causal masking is not an optimisation here").
 *   - d must be 64 or 128. N >= 1; N * d must not exceed 2^30.
 *   - Ownership: the caller allocates and frees every buffer, including workspaces. The library
 *     allocates no device memory, keeps no pointer after a call returns, and holds no state except
 *     the opt-in kernel timer below and, per device, whether it has already raised a kernel's
 *     dynamic-LDS limit (done on a kernel's first launch on that device). Calls from several host
 *     threads may run concurrently, on different streams and buffers; the timer is the exception.
 *   - Execution: work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call
 *     returns without waiting. Faults inside a kernel surface at the caller's next synchronisation.
 *   - Errors: every argument check runs before any launch; a failing check enqueues nothing and
 *     returns a non-zero attn_status. attn_last_error() then describes it (per calling thread).
 *     Output buffers must not overlap input buffers (checked by address range).
 */
#ifndef ROOFLINE_ATTENTION_ATTN_H
#define ROOFLINE_ATTENTION_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, overlap, H % H_kv != 0 */
  ATTN_ERR_UNSUPPORTED = 2, /* d not in {64, 128}, dtype not supported by this entry point */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query returns */
  ATTN_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} attn_status;

typedef enum attn_dtype {
  ATTN_F32 = 0,  /* float32 storage and arithmetic */
  ATTN_BF16 = 1  /* bfloat16 storage, float32 accumulation */
} attn_dtype;

/* Version of this ABI; bumped on any signature or semantic change. */
int attn_abi_version(void);

/* Static name of a status code (never NULL). */
const char* attn_status_string(int status);

/* Message describing the last failing call made by this thread ("" if none). */
const char* attn_last_error(void);

/*
 * Forward pass (prefill): O = softmax(scale * Q K^T [causal]) V and, if lse != NULL, LSE.
 *   dtype ATTN_F32 : q, k, v, o are float32.
 *   dtype ATTN_BF16: q, k, v, o are bfloat16 (o rounded to nearest even); lse is float32.
 * The online-softmax recurrence (running row maximum and normaliser, output rescaled as each
 * K/V block arrives) follows "Why Fast GPUs Still Wait for Memory", section "FlashAttention is an
 * IO algorithm"; it equals the two-pass softmax up to rounding.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int H_kv, int N, int d, int causal, float scale,
                     int dtype, void* stream);

/*
 * fp8 forward: the same attention for inputs stored as 8-bit floats, which double the matrix-core
 * ceiling ("Why Fast GPUs Still Wait for Memory", section "pi is the top of a stack" and Table 1:
 * fp8 doubles pi and the ridge point). The pages leave the format and its scaling metadata open;
 * this entry point takes OCP FP8 E4M3 codes (exponent bias 7, no infinities, S.1111.111 = NaN,
 * largest finite 448) with one float32 descale factor per tensor:
 *   real Q = q_descale * decode(q), real K = k_descale * decode(k), real V = v_descale * decode(v),
 *   O = softmax(scale * Q K^T [causal]) V of those real values, LSE as for attn_fwd.
 *   q [B, H, N, d], k, v [B, H_kv, N, d]: uint8 codes; o [B, H, N, d] bfloat16 (nearest even);
 *   lse [B, H, N] float32 or NULL. d must be 64 or 128. Descales must be finite (any sign or zero).
 * Accuracy: scores are exact products of the codes accumulated in float32; the probabilities that
 * multiply V are rounded to E4M3 (relative error at most 2^-4 each, values below 2^-12 of the row
 * maximum with an absolute error of at most 2^-16 of it), while the normaliser and LSE use the
 * unrounded float32 probabilities. NaN codes propagate to the rows they reach.
 */
attn_status attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int H_kv, int N, int d, int causal, float scale,
                         float q_descale, float k_descale, float v_descale, void* stream);

/*
 * Ragged (variable-length) prefill: B sequences of different lengths packed row after row, with
 * no padding. A padded batch of ragged sequences runs partly empty ("Why Fast GPUs Still Wait for
 * Memory", section "Shapes matter", trap "B* is not a batch size you can actually run"); here each
 * workgroup covers query rows of one sequence only. Each sequence is computed exactly as attn_fwd
 * computes one (batch) entry: it attends only to its own rows, and causal positions count from
 * its first row.
 *   q, o [T, H, d] bf16; k, v [T, H_kv, d] bf16 (row t of every head contiguous, d innermost);
 *   lse [H, T] float32 natural log, or NULL; cu_seqlens [B + 1] int32 DEVICE array, sequence b is
 *   rows cu_seqlens[b] .. cu_seqlens[b+1] - 1, with cu_seqlens[0] = 0, non-decreasing, and
 *   cu_seqlens[B] = T. max_seqlen >= every sequence length (it sizes the grid). The kernel clamps
 *   offsets into [0, T] and lengths to max_seqlen, so malformed offsets cannot make it access
 *   memory outside the tensors, but the results are then unspecified; rows of an empty sequence
 *   are simply absent. T == 0 returns ATTN_OK without device work.
 * dtype must be ATTN_BF16; d in {64, 128}; H % H_kv == 0.
 */
attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens, int B, int max_seqlen, int T, int H, int H_kv, int d,
                            int causal, float scale, int dtype, void* stream);

/*
 * Decode: one query token per (sequence, head) against a KV cache, the regime of
 * "Why Fast GPUs Still Wait for Memory", section "Attention III - KV cache, GQA, MLA"
 * (I = 2g/s, memory-bound). The keys of all sequences are split across workgroups in equal
 * shares (a share may cover parts of several sequences) and a second kernel merges the partial
 * (max, sum, output) triples ("M4.2 - GPU Execution Model for Transformer Kernels", section 0x08:
 * split-K needs an extra reduction).
 *   q [B, H, d] bf16; k_cache, v_cache [B, H_kv, N_cap, d] bf16; o [B, H, d] bf16;
 *   lse [B, H] float32 or NULL; kv_len [B] int32 DEVICE array, sequence b attends to cache rows
 *   0 .. kv_len[b]-1 and never reads rows at or beyond kv_len[b]. Values are clamped to
 *   [0, N_cap] on the device; kv_len[b] == 0 yields o = 0 and lse = -inf for that sequence.
 *   `causal` is accepted for signature symmetry and ignored: the single query follows every key.
 *   workspace: device buffer of at least attn_decode_workspace_size(B, H, N_cap, d) bytes,
 *   16-byte aligned, contents need no initialisation; it is scratch owned by the caller.
 * dtype must be ATTN_BF16. Any group size g = H / H_kv: g = 1, 2, 4, 8 have kernels of their own;
 * other g run a 16-column kernel over chunks of up to 16 query heads (for g > 16 each chunk reads
 * the KV head's rows again). B * H_kv * (g in {1,2,4,8} ? 1 : ceil(g / 16)) must be below 2^24.
 */
size_t attn_decode_workspace_size(int B, int H, int N_cap, int d);
attn_status attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                        const int32_t* kv_len, int B, int H, int H_kv, int N_cap, int d, int causal,
                        float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode with no allocation and no workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same operation, arguments (less the workspace) and results as attn_decode, bit for bit: the
 * split records live in a fixed scratch array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends. The call makes no hipMalloc, hipFree or other
 * allocating call (with the opt-in timer below off: its events are its only objects); the first
 * call on a device looks up the array's address there (hipGetSymbolAddress) and caches it.
 * Shapes whose attn_decode_workspace_size(B, H, N_cap, d) exceeds the scratch are rejected with
 * ATTN_ERR_WORKSPACE before any device work. Every call on one GPU shares that GPU's scratch, so
 * calls that overlap in time on one GPU (other streams, other host threads) race and give wrong
 * results; calls ordered on one stream are safe. The scratch needs no initial contents.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
attn_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                const int32_t* kv_len, int B, int H, int H_kv, int N_cap, int d, int causal,
                                float scale, int dtype, void* stream);

/*
 * Decode over a paged KV cache: as attn_decode, but the cache lives in fixed-size pages that need
 * not be contiguous or in order. A kernel's contract has to state the page layout when K/V is not
 * contiguous ("M4.2 - GPU Execution Model for Transformer Kernels", section 0x06), and logical
 * K/V continuity does not imply contiguous physical addresses (same page, section 0x0D, failure 16).
 *   k_pages, v_pages [num_pages, H_kv, page_size, d] bf16: page p holds page_size consecutive cache
 *   rows of every KV head, rows of one head contiguous. block_table [B, max_pages] int32 DEVICE
 *   array: cache row j of sequence b is row j % page_size of page block_table[b][j / page_size].
 *   kv_len [B] int32 DEVICE array, clamped to [0, max_pages * page_size] on the device; only
 *   the table entries of rows below kv_len[b] are used. Page ids are clamped into [0, num_pages)
 *   on the device, so a malformed table cannot make the kernel read outside the pages (the result
 *   is then unspecified).
 *   page_size: a power of two in [32, 1024] (a 32-key tile then never straddles a page).
 *   workspace: at least attn_decode_workspace_size(B, H, max_pages * page_size, d) bytes.
 * dtype must be ATTN_BF16; group sizes and the grid limit as for attn_decode.
 */
attn_status attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse,
                              const int32_t* kv_len, const int32_t* block_table, int B, int H, int H_kv,
                              int num_pages, int page_size, int max_pages, int d, float scale, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass: gradients of L = sum(O * dO) with respect to Q, K and V, recomputing the scores
 * from Q and K instead of reading a stored N x N matrix ("Why Fast GPUs Still Wait for Memory",
 * section "FlashAttention is an IO algorithm": the backward recomputes S). Every gradient element
 * is written by exactly one workgroup and no atomics are used (the race-free-by-construction rule
 * of the MoA paper, "Validating Memory-Optimal Transformer Kernels on Real Hardware", section 4.5).
 *   q, k, v, o, dout: bf16 in the layouts above; o and lse must come from attn_fwd on the same
 *   q, k, v, causal and scale. dq [B,H,N,d], dk, dv [B,H_kv,N,d]: float32, fully overwritten.
 *   Grouped heads (H_kv < H, H % H_kv == 0): the dK/dV of a KV head sum the contributions of its
 *   H / H_kv query heads, accumulated by the one workgroup that owns those rows (no K/V expansion,
 *   "Why Fast GPUs Still Wait for Memory", section "Attention III - KV cache, GQA, MLA").
 *   workspace: at least attn_bwd_workspace_size(B, H, N, d) bytes, 16-byte aligned, scratch.
 * dtype must be ATTN_BF16.
 */
size_t attn_bwd_workspace_size(int B, int H, int N, int d);
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, float* dq, float* dk, float* dv,
                     int B, int H, int H_kv, int N, int d, int causal, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Ragged backward: attn_bwd over the packed rows of attn_fwd_varlen. Sequences share no score, so
 * each sequence's gradients are those attn_bwd computes for one (batch) entry of its length, with
 * causal positions counted from its first row; the same two atomic-free kernels run over the
 * packed rows, each workgroup covering one sequence's rows.
 *   q, o, dout [T, H, d] bf16; k, v [T, H_kv, d] bf16; lse [H, T] float32 from attn_fwd_varlen on
 *   the same q, k, v, cu_seqlens, causal and scale. dq [T, H, d], dk, dv [T, H_kv, d] float32:
 *   every row of every sequence is overwritten. cu_seqlens, max_seqlen, T and the clamping of
 *   malformed offsets as for attn_fwd_varlen; T == 0 returns ATTN_OK without device work.
 *   workspace: at least attn_bwd_varlen_workspace_size(T, H, d) bytes, 16-byte aligned, scratch.
 * dtype must be ATTN_BF16; d in {64, 128}; H % H_kv == 0.
 */
size_t attn_bwd_varlen_workspace_size(int T, int H, int d);
attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, float* dq, float* dk, float* dv, const int32_t* cu_seqlens,
                            int B, int max_seqlen, int T, int H, int H_kv, int d, int causal, float scale,
                            int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward and backward in ONE launch, with no atomic accumulation: the fused forward+backward of
 * the MoA paper ("Validating Memory-Optimal Transformer Kernels on Real Hardware", sections
 * 4.4-4.5), whose GPU version lost to the unfused pair while dK and dV were accumulated with atomics
 * and won once every gradient element had a single owner. Computes what attn_fwd followed by
 * attn_bwd compute (o, lse, and the gradients of L = sum(O * dO)), as one cooperative kernel: a
 * first phase runs the forward of each query tile together with that tile's dQ, a grid barrier
 * follows, and a second phase computes dK and dV per key tile.
 *   q, dout [B,H,N,d], k, v [B,H_kv,N,d]: bfloat16 inputs. Outputs, fully overwritten: o [B,H,N,d]
 *   bfloat16, lse [B,H,N] float32 (required), dq [B,H,N,d], dk, dv [B,H_kv,N,d] float32.
 *   workspace: at least attn_fwd_bwd_workspace_size(B, H, N, d) bytes, 16-byte aligned, scratch
 *   owned by the caller (contents need no initialisation). Calls that share a workspace must not
 *   run concurrently.
 * dtype must be ATTN_BF16. The launch needs the device's cooperative-launch support; it returns
 * ATTN_ERR_HIP if the runtime refuses it.
 */
size_t attn_fwd_bwd_workspace_size(int B, int H, int N, int d);
attn_status attn_fwd_bwd(const void* q, const void* k, const void* v, const void* dout, void* o, float* lse,
                         float* dq, float* dk, float* dv, int B, int H, int H_kv, int N, int d, int causal,
                         float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Opt-in kernel timer for measurement harnesses ("M4.2 - GPU Execution Model for Transformer
 * Kernels", section 0x0B: device-side timing with events on the launching stream). While enabled,
 * every kernel the library launches is bracketed by a pair of HIP events on its own stream.
 * attn_timing_get synchronises on the recorded events and returns, for the index-th kernel name
 * seen since the last reset, its static name, launch count and summed duration in milliseconds.
 * Not for concurrent use from several threads.
 */
attn_status attn_timing_enable(int on);
attn_status attn_timing_reset(void);
int attn_timing_count(void);
attn_status attn_timing_get(int index, const char** name, long long* launches, double* total_ms);

/*
 * Per-launch durations behind attn_timing_get, so a harness can report a distribution (median and
 * tail percentiles, "M4.2 - GPU Execution Model for Transformer Kernels", section 0x0B, Level 4)
 * instead of one mean: writes the durations in milliseconds of the first min(cap, launches)
 * launches of the index-th kernel name, in launch order, to ms[0..cap) (host memory owned by the
 * caller) and returns the number of launches recorded since the last reset. Returns -1 on a bad
 * index, on cap < 0, on ms == NULL with cap > 0, or on a HIP error (attn_last_error says which).
 */
int attn_timing_samples(int index, float* ms, int cap);

/*
 * Releases every HIP object the library has created: it disables the timer, waits for the events
 * still pending and destroys all timing events (the only objects the library creates; it
 * allocates no device memory). Meant for the end of a process, so that no library-owned runtime
 * object is left to the HIP runtime's own teardown (where a tool that intercepts HIP calls, such
 * as a profiler, may already have finalised). The library stays usable afterwards: a later timed
 * launch creates events again. Not for concurrent use with timed launches.
 */
attn_status attn_release(void);

#ifdef __cplusplus
}
#endif

#endif /* ROOFLINE_ATTENTION_ATTN_H */
