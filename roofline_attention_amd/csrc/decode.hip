// Split-KV decode attention for one query token per (sequence, head) over a bf16 KV cache.
//
// Decode is memory-bound at I = 2g/s FLOP/byte for group size g ("Why Fast GPUs Still Wait for
// Memory", section "Attention III - KV cache, GQA, MLA"), so the kernel is built to stream K and V
// at HBM rate: every K/V byte is read once, and all g query heads of a KV head are served from
// the same bytes (the grouped physical path, no K/V expansion). The key axis is split into
// fixed-size chunks, one workgroup each, so ragged sequence lengths never leave a long serial tail;
// the partial (max, sum, output) triples are merged by a second kernel ("M4.2 - GPU Execution
// Model for Transformer Kernels", section 0x08: split-K trades parallelism for an extra
// reduction pass).
//
// Split kernel, one 4-wave workgroup per (1024-key split, KV head, sequence); within a wave,
//   lane = (key slot ks, 16-byte chunk dc of the head dimension). One load instruction covers
//   KPI consecutive cache rows (contiguous bytes), the partial dot products are joined across the
//   chunk lanes with DPP, and the softmax is kept online over sub-chunks of ITERS * KPI keys whose
//   loads are issued one sub-chunk ahead. The partial record of each query head is
//   {m, l, -, -, o[d]} with m in log2 units of the scaled score and o not yet divided by l.
// Combine kernel, one wave per (query head, sequence): M = max m_s, L = sum 2^(m_s - M) l_s,
//   O = sum 2^(m_s - M) o_s / L, LSE = ln 2 * (M + log2 L).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace ra {
namespace {


constexpr int DEC_WAVES = 4;                             // waves per workgroup
constexpr int DEC_WAVE_KEYS = kDecodeSplit / DEC_WAVES;  // keys per wave (256)
constexpr int DEC_TILE = 32;                             // keys per LDS stage
constexpr int DEC_STAGES = 2;

__device__ __forceinline__ int clamp_len(const int32_t* kv_len, int b, int N_cap) {
  const int len = kv_len[b];
  return len < 0 ? 0 : (len > N_cap ? N_cap : len);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Per-wave LDS: DEC_STAGES stages of a DEC_TILE-key K tile and V tile, unpadded rows with the
// 16-byte chunk c of row r at position c ^ swz(r). K is read as MFMA A-operand rows (16 rows, one
// chunk per 16-lane group: swz_k = r mod CH); V by transposed reads (8 rows x 2 chunks per 32
// lanes: swz_v = 2r mod CH).
template <int HD>
struct DecodeWaveSmem {
  bf16 k[DEC_STAGES][DEC_TILE * HD];
  bf16 v[DEC_STAGES][DEC_TILE * HD];
};

template <int HD, int G>
struct DecodeMerge {
  float m[DEC_WAVES][G];
  float l[DEC_WAVES][G];
  float o[DEC_WAVES][G][HD];
};

template <int HD>
constexpr size_t decode_smem_bytes(int G) {
  const size_t stages = sizeof(DecodeWaveSmem<HD>) * DEC_WAVES;
  const size_t merge = (size_t)DEC_WAVES * G * (HD + 2) * sizeof(float);
  return stages > merge ? stages : merge;
}


// One workgroup = 4 waves over kDecodeSplit consecutive keys of one (sequence, KV head); wave w
// takes keys [256w, 256w + 256) of the split and works independently of the other waves until
// the final merge. Per 32-key tile (HBM -> LDS by buffer_load ... lds, two stages in flight):
//   S^T = K Q^T on 16x16x32 MFMAs (A = 16 keys x 32 d from LDS, B = the g query heads of the KV
//   head as columns, padded with zero columns to 16), online softmax per head on the few lanes
//   that hold real heads, O^T += V^T P^T on 16x16x32 MFMAs with V^T from transposed LDS reads.
// The matrix cores do the dot products that would otherwise cost several vector ops per byte;
// the vector ALUs only run the softmax of 32 keys x g heads per tile.
template <int HD, int G>
__global__ __launch_bounds__(DEC_WAVES * 64) void decode_split_kernel(
    const bf16* __restrict__ Qd, const bf16* __restrict__ Kc, const bf16* __restrict__ Vc,
    const int32_t* __restrict__ kv_len, float* __restrict__ ws, int H, int H_kv, int N_cap,
    int n_split, float scale_log2) {
  constexpr int CH = HD / 8;        // 16-byte chunks per row
  constexpr int KSTEPS = HD / 32;   // 16x16x32 k-steps over d
  constexpr int CB = HD / 16;       // 16-row blocks of O^T
  constexpr int RPI = 1024 / (HD * 2);       // rows per direct-load instruction
  constexpr int LOADS = DEC_TILE / RPI;      // instructions per tensor per tile
  constexpr int REC = HD + 4;
  static_assert(G <= 16, "query heads per KV head");
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];

  const int split = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int len = clamp_len(kv_len, b, N_cap);
  const int k_begin = split * kDecodeSplit;
  if (k_begin >= len) return;  // uniform over the workgroup, before any barrier

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;  // MFMA column = query head of the group (valid when < G)
  const int q4 = lane >> 4;   // 16-lane group
  const int kw_begin = k_begin + w * DEC_WAVE_KEYS;
  const int kw_end = min(len, kw_begin + DEC_WAVE_KEYS);
  const int n_keys = max(kw_end - kw_begin, 0);
  const int n_tiles = (n_keys + DEC_TILE - 1) / DEC_TILE;
  DecodeWaveSmem<HD>& sm = reinterpret_cast<DecodeWaveSmem<HD>*>(dyn_smem)[w];

  // Q^T as the B operand: column col = head hk*G + col, k-group q4 holds d = 32kk + 8q4 .. +7.
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    qf[kk] = col < G ? *reinterpret_cast<const bf16x8*>(Qd + ((size_t)b * H + hk * G + col) * HD + 32 * kk + 8 * q4)
                     : bf16x8{};
  }

  const size_t head = ((size_t)b * H_kv + hk) * (size_t)N_cap * HD;
  // Resources over this wave's keys only: rows at or past kw_end load as zeros.
  const auto krs = make_rsrc(Kc + head + (size_t)kw_begin * HD, n_keys * HD * 2);
  const auto vrs = make_rsrc(Vc + head + (size_t)kw_begin * HD, n_keys * HD * 2);
  const int st_row = lane / CH;
  auto issue = [&](int t) {
    const int stage = t % DEC_STAGES;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int row = u * RPI + st_row;
      const int kvo = (row * HD + (((lane % CH) ^ (row & (CH - 1))) * 8)) * 2;
      const int vvo = (row * HD + (((lane % CH) ^ ((2 * row) & (CH - 1))) * 8)) * 2;
      const int toff = t * DEC_TILE * HD * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void_ptr)(&sm.k[stage][u * RPI * HD]), 16, toff + kvo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void_ptr)(&sm.v[stage][u * RPI * HD]), 16, toff + vvo, 0, 0, 0);
    }
  };

  // K A-operand: row key = 16*half + col, chunk 4kk + q4 at position ^ swz_k(row).
  // V^T A-operand (transposed read): in 16-lane group q4, source lane 4e + j points at key row
  // base + 4*q4 + e and column 16cb + 4j; the lane receives column 16cb + col of 4 keys.
  const int v_e = (lane & 15) >> 2;
  const int v_j = lane & 3;

  f32x4 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = scale_log2;

  if (n_tiles > 0) issue(0);
  if (n_tiles > 1) issue(1);
  for (int t = 0; t < n_tiles; ++t) {
    if (t + 1 < n_tiles)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LOADS));  // only the next tile's loads may be in flight
    else
      __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");  // LDS reads of this tile stay after the wait
    const int stage = t % DEC_STAGES;
    const bf16* kt = sm.k[stage];
    const bf16* vt = sm.v[stage];
    // S^T for keys 16*half + 4*q4 + r (r = 0..3), column = head.
    f32x4 s[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      s[half] = f32x4{};
      const int row = 16 * half + col;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + row * HD + (((4 * kk + q4) ^ (row & (CH - 1))) * 8));
        s[half] = mfma16(a, qf[kk], s[half]);
      }
    }
    const int key0 = t * DEC_TILE;  // relative to kw_begin
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + 16 * half + 4 * q4 + r;
        const float v = key < n_keys ? s[half][r] * c : -INFINITY;
        x[4 * half + r] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    // Tile 0 holds the wave's first key, so m_run is finite after it.
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    bf16x8 pb;
    float tsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(x[e] - m_new);
      tsum += p;
      pb[e] = to_bf16(p);
    }
    l_run = fmaf(l_run, alpha, tsum);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
    }
    // O^T += V^T P^T: k-slot e < 4 is key 4*q4 + e, e >= 4 is key 16 + 4*q4 + (e - 4).
    bf16x8 va[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const bf16* p0 = vt + (4 * q4 + v_e) * HD;
      const bf16* p1 = vt + (16 + 4 * q4 + v_e) * HD;
      const int c0 = ((2 * cb + (v_j >> 1)) ^ ((2 * (4 * q4 + v_e)) & (CH - 1))) * 8 + 4 * (v_j & 1);
      const int c1 = ((2 * cb + (v_j >> 1)) ^ ((2 * (16 + 4 * q4 + v_e)) & (CH - 1))) * 8 + 4 * (v_j & 1);
      va[cb] = tr_pair_async(p0 + c0, p1 + c1);
    }
    lds_wait_all(va);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[cb] = mfma16(va[cb], pb, acc[cb]);
    if (t + 2 < n_tiles) {
      // The stage just consumed is refilled: its LDS reads must have completed first.
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt at their maxima
      asm volatile("" ::: "memory");
      issue(t + 2);
    }
  }

  // l: each lane summed its 8 keys per tile; the 4 lanes of a head column hold the rest.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  __syncthreads();  // every wave is done with its stages; the merge area overlays them
  DecodeMerge<HD, G>& mg = *reinterpret_cast<DecodeMerge<HD, G>*>(dyn_smem);
  if (col < G) {
    if (q4 == 0) {
      mg.m[w][col] = m_run;  // -inf for a wave with no keys
      mg.l[w][col] = l_run;
    }
    // O^T rows c = 16cb + 4*q4 + r of head column col.
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      *reinterpret_cast<f32x4*>(&mg.o[w][col][16 * cb + 4 * q4]) = acc[cb];
  }
  __syncthreads();
  constexpr int PER = HD / 64;
  for (int hq = w; hq < G; hq += DEC_WAVES) {
    float M = mg.m[0][hq];  // wave 0 always has keys
#pragma unroll
    for (int v = 1; v < DEC_WAVES; ++v) M = fmaxf(M, mg.m[v][hq]);
    float L = 0.f, o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
    for (int v = 0; v < DEC_WAVES; ++v) {
      const float wgt = fast_exp2(mg.m[v][hq] - M);  // 0 for a wave with no keys
      L = fmaf(wgt, mg.l[v][hq], L);
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] = fmaf(wgt, mg.o[v][hq][lane * PER + e], o[e]);
    }
    float* rec = ws + (((size_t)b * H + hk * G + hq) * n_split + split) * REC;
    if (lane == 0) {
      rec[0] = M;
      rec[1] = L;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) rec[4 + lane * PER + e] = o[e];
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
  const size_t smem = decode_smem_bytes<HD>(G);
  static bool attr_set = false;  // one dynamic-LDS opt-in per instantiation
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_split_kernel<HD, G>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  {
    TimedScope ts(split_name, stream);
    hipLaunchKernelGGL((decode_split_kernel<HD, G>), dim3(n_split, H_kv, B), dim3(DEC_WAVES * 64), smem, stream,
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
