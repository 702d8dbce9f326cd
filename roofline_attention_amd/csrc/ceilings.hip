// Ceiling microbenchmarks for the MI355X roofline the attention kernels are measured against.
//
// "Why Fast GPUs Still Wait for Memory" (section "pi is the top of a stack") warns that the
// published peak is the top of a stack of lower ceilings that depend on the instruction mix. This
// program measures the ceilings the kernels here actually run into, on the machine at hand:
//   mfma_bf16 / mfma_fp8: full-chip rate of independent v_mfma_f32_32x32x16_bf16 and
//                         v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3), in TFLOP/s (timed with events),
//                         and the cycles one instruction occupies the matrix pipe (clock64, one
//                         wave per SIMD); the *_random variants feed operands like real data;
//   hbm_read, hbm_copy:   streaming read (sum of a 2 GiB buffer, non-temporal 16-byte loads,
//                         8 workgroups per CU, grid-stride) and copy, in GB/s;
//   lds_read:             bytes per clock per CU for ds_read_b128 and ds_read_b64_tr_b16;
//   valu:                 cycles per wave instruction of v_fma_f32 and v_exp_f32;
//   coexec:               8 waves per workgroup (two per SIMD): all MFMA, all VALU, MFMA waves beside
//                         VALU waves, and every wave interleaving its own MFMAs and VALU — whether a
//                         vector instruction overlaps another wave's MFMA.
// Output: one JSON line on stdout. Every kernel stays inside its own buffers and LDS arrays.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

#define CHECK(x)                                                                  \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                    \
    }                                                                             \
  } while (0)

// Calls launch() until 0.2 s of wall time have passed, synchronising every 8 launches.
template <class F>
void warm_up(F launch) {
  const auto t0 = std::chrono::steady_clock::now();
  for (int n = 1;; ++n) {
    launch();
    if (n % 8 == 0) {
      CHECK(hipDeviceSynchronize());
      if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(200)) break;
    }
  }
}

// ----------------------------------------------------------------------------------- MFMA ----

constexpr int MFMA_IT = 4000;

// KIND 0: bf16 32x32x16, 1: E4M3 32x32x64, both on operands that are the same small values in every
// lane and every instruction; 2 and 3: the same instructions on operands like the attention kernels'
// (per lane pseudo-random values with full mantissas, a different operand pair for each of eight
// consecutive instructions), which switch far more of the matrix datapath: under the chip's power
// management the clock, and with it the rate, depends on the data.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_kernel(float* out, unsigned long long* cyc, int seed) {
  constexpr bool RANDOM = KIND >= 2;
  constexpr bool FP8 = KIND == 1 || KIND == 3;
  constexpr int SETS = RANDOM ? 8 : 1;
  f32x16 acc[4] = {};
  bf16x8 a[SETS], b[SETS];
  i32x8 wa[SETS], wb[SETS];
  uint32_t x = (uint32_t)seed * 2654435761u ^ (uint32_t)(blockIdx.x * 256 + threadIdx.x + 1) * 0x9E3779B9u;
  auto next = [&]() {  // xorshift32
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
  };
  for (int j = 0; j < SETS; ++j) {
    for (int i = 0; i < 8; ++i) {
      if constexpr (RANDOM) {
        // uniform in [-2, 2) with a full 8-bit mantissa; E4M3 codes with random sign, exponent
        // 4..11 and mantissa (finite, no NaN code)
        a[j][i] = (__bf16)((float)((int)(next() & 0xffff) - 32768) * (1.f / 16384.f));
        b[j][i] = (__bf16)((float)((int)(next() & 0xffff) - 32768) * (1.f / 16384.f));
        uint32_t ca = 0, cb = 0;
        for (int byte = 0; byte < 4; ++byte) {
          const uint32_t r1 = next(), r2 = next();
          ca |= ((r1 & 0x80) | (((r1 >> 8) & 7) + 4) << 3 | ((r1 >> 16) & 7)) << (8 * byte);
          cb |= ((r2 & 0x80) | (((r2 >> 8) & 7) + 4) << 3 | ((r2 >> 16) & 7)) << (8 * byte);
        }
        wa[j][i] = (int)ca;
        wb[j][i] = (int)cb;
      } else {
        a[j][i] = (__bf16)(float)((seed + i) & 3);
        b[j][i] = (__bf16)(float)((i - seed) & 3);
        wa[j][i] = 0x38383838 + i;
        wb[j][i] = 0x38383838 - i;
      }
    }
  }
  const unsigned long long t0 = clock64();
  for (int it = 0; it < MFMA_IT / SETS * SETS; it += SETS) {
#pragma unroll
    for (int j = 0; j < SETS; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int o = (j + q) % SETS;  // a different operand pair for each of the four chains
        if constexpr (!FP8) acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[o], b[o], acc[q], 0, 0, 0);
        else acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa[o], wb[o], acc[q], 0, 0, 0, 127, 0, 127);
      }
    }
  }
  const unsigned long long t1 = clock64();
  float s = 0.f;
  for (int q = 0; q < 4; ++q) s += acc[q][threadIdx.x & 15];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) cyc[blockIdx.x] = t1 - t0;
}

template <int KIND>
void mfma_rate(int cus, double& tflops, double& cycles_per_inst) {
  const int grid = cus;  // one workgroup of four waves per CU: one wave per SIMD
  float* out;
  unsigned long long* cyc;
  CHECK(hipMalloc(&out, (size_t)grid * 256 * 4));
  CHECK(hipMalloc(&cyc, (size_t)grid * 8));
  // Untimed launches for 0.2 s first: the clock takes tens of milliseconds of load to ramp up.
  warm_up([&] { hipLaunchKernelGGL(mfma_kernel<KIND>, dim3(grid), dim3(256), 0, 0, out, cyc, 3); });
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  constexpr int kTimed = 10;
  CHECK(hipEventRecord(e0));
  for (int i = 0; i < kTimed; ++i) hipLaunchKernelGGL(mfma_kernel<KIND>, dim3(grid), dim3(256), 0, 0, out, cyc, 3);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  unsigned long long c0 = 0;
  CHECK(hipMemcpy(&c0, cyc, 8, hipMemcpyDeviceToHost));
  const double flops_per_inst = (KIND == 0 || KIND == 2) ? 2.0 * 32 * 32 * 16 : 2.0 * 32 * 32 * 64;
  const double insts = (double)kTimed * grid * 4 /* waves */ * MFMA_IT * 4;
  tflops = insts * flops_per_inst / (ms * 1e-3) / 1e12;
  // one wave per SIMD issuing independent MFMAs: cycles between its instructions = pipe occupancy
  cycles_per_inst = (double)c0 / (MFMA_IT * 4);
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
}

// ------------------------------------------------------------------------------------ HBM ----

__global__ __launch_bounds__(256) void read_kernel(const f4* __restrict__ src, size_t n, float* out) {
  f4 acc = {0, 0, 0, 0};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const f4 v = __builtin_nontemporal_load(&src[i]);
    acc += v;
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc[0] + acc[1] + acc[2] + acc[3];
}

__global__ __launch_bounds__(256) void copy_kernel(const f4* __restrict__ src, f4* __restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}

void hbm(int cus, double& read_gbs, double& copy_gbs) {
  const size_t bytes = (size_t)2 << 30;
  const size_t n = bytes / 16;
  f4 *a, *b;
  float* out;
  const int grid = cus * 8;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMalloc(&out, (size_t)grid * 256 * 4));
  CHECK(hipMemset(a, 0, bytes));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float best_r = 1e30f, best_c = 1e30f;
  warm_up([&] { hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, 0, a, n, out); });
  for (int rep = 0; rep < 6; ++rep) {
    float ms = 0.f;
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, 0, a, n, out);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (rep > 0 && ms < best_r) best_r = ms;
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, 0, a, b, n);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (rep > 0 && ms < best_c) best_c = ms;
  }
  read_gbs = (double)bytes / (best_r * 1e-3) / 1e9;
  copy_gbs = 2.0 * (double)bytes / (best_c * 1e-3) / 1e9;
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  CHECK(hipFree(out));
}

// ------------------------------------------------------------------------------------ LDS ----

constexpr int LDS_IT = 4096;

template <int KIND>  // 0: ds_read_b128, 1: ds_read_b64_tr_b16 (conflict-free addresses)
__global__ __launch_bounds__(256) void lds_kernel(unsigned long long* cyc, float* sink) {
  __shared__ __attribute__((aligned(16))) float lds[16384];  // 64 KB
  for (int i = threadIdx.x; i < 16384; i += 256) lds[i] = (float)(i & 7);
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // each wave reads its own 16 KB quarter; offsets stay below 16 KB - 16 within it
  const unsigned base =
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) float*)&lds[w * 4096] + lane * (KIND == 0 ? 16 : 8);
  float acc = 0.f;
  const unsigned long long t0 = clock64();
  for (int it = 0; it < LDS_IT; ++it) {
    if constexpr (KIND == 0) {
      f4 x, y, z, u;
      asm volatile(
          "ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:1024\n ds_read_b128 %2, %4 offset:2048\n"
          " ds_read_b128 %3, %4 offset:3072\n s_waitcnt lgkmcnt(0)"
          : "=v"(x), "=v"(y), "=v"(z), "=v"(u)
          : "v"(base));
      acc += x[0] + y[1] + z[2] + u[3];
    } else {
      f2 x, y, z, u, p, q, r, s;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n ds_read_b64_tr_b16 %1, %8 offset:512\n ds_read_b64_tr_b16 %2, %8 offset:1024\n"
          " ds_read_b64_tr_b16 %3, %8 offset:1536\n ds_read_b64_tr_b16 %4, %8 offset:2048\n"
          " ds_read_b64_tr_b16 %5, %8 offset:2560\n ds_read_b64_tr_b16 %6, %8 offset:3072\n"
          " ds_read_b64_tr_b16 %7, %8 offset:3584\n s_waitcnt lgkmcnt(0)"
          : "=v"(x), "=v"(y), "=v"(z), "=v"(u), "=v"(p), "=v"(q), "=v"(r), "=v"(s)
          : "v"(base));
      acc += x[0] + y[1] + z[0] + u[1] + p[0] + q[1] + r[0] + s[1];
    }
  }
  const unsigned long long t1 = clock64();
  if (lane == 0) cyc[blockIdx.x * 4 + w] = t1 - t0;
  sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

template <int KIND>
double lds_bytes_per_clk(int cus) {
  const int grid = cus * 2;  // two workgroups (8 waves) per CU
  unsigned long long* cyc;
  float* sink;
  CHECK(hipMalloc(&cyc, (size_t)grid * 4 * 8));
  CHECK(hipMalloc(&sink, (size_t)grid * 256 * 4));
  hipLaunchKernelGGL(lds_kernel<KIND>, dim3(grid), dim3(256), 0, 0, cyc, sink);
  hipLaunchKernelGGL(lds_kernel<KIND>, dim3(grid), dim3(256), 0, 0, cyc, sink);
  CHECK(hipDeviceSynchronize());
  unsigned long long c = 0;
  CHECK(hipMemcpy(&c, cyc, 8, hipMemcpyDeviceToHost));
  // bytes moved by the 8 waves of a CU while one of them ran c cycles
  const double bytes = 8.0 * LDS_IT * (KIND == 0 ? 4 * 1024.0 : 8 * 512.0);
  CHECK(hipFree(cyc));
  CHECK(hipFree(sink));
  return bytes / (double)c;
}

// ------------------------------------------------------------------------------ VALU rate ----

constexpr int VALU_IT = 4000;

template <int KIND>  // 0: v_fma_f32, 1: v_exp_f32
__global__ __launch_bounds__(64) void valu_kernel(float* out, unsigned long long* cyc, float seed) {
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = seed * (i + 1) * 1e-3f + threadIdx.x * 1e-6f;
  const unsigned long long t0 = clock64();
  for (int it = 0; it < VALU_IT; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (KIND == 0) x[i] = __builtin_fmaf(x[i], 0.999f, 1e-3f);
      else x[i] = __builtin_amdgcn_exp2f(x[i] * -0.5f);
    }
  }
  const unsigned long long t1 = clock64();
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += x[i];
  out[threadIdx.x] = s;
  if (threadIdx.x == 0) cyc[0] = t1 - t0;
}

template <int KIND>
double valu_cycles() {
  float* out;
  unsigned long long* cyc;
  CHECK(hipMalloc(&out, 64 * 4));
  CHECK(hipMalloc(&cyc, 8));
  hipLaunchKernelGGL(valu_kernel<KIND>, dim3(1), dim3(64), 0, 0, out, cyc, 0.5f);
  hipLaunchKernelGGL(valu_kernel<KIND>, dim3(1), dim3(64), 0, 0, out, cyc, 0.5f);
  CHECK(hipDeviceSynchronize());
  unsigned long long c = 0;
  CHECK(hipMemcpy(&c, cyc, 8, hipMemcpyDeviceToHost));
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  // x * -0.5 costs one multiply per exponential (a separate instruction)
  return (double)c / (VALU_IT * 16.0) - (KIND == 1 ? valu_cycles<0>() : 0.0);
}

// --------------------------------------------------------------------------- co-execution ----

constexpr int CO_IT = 2000;

// mode 0: every wave MFMA only; 1: every wave VALU only; 2: waves 0-3 MFMA, waves 4-7 VALU (each SIMD
// runs one of each); 3: every wave interleaves its own MFMAs and VALU. Per iteration a wave issues
// 4 MFMAs (~128 pipe cycles) and/or 32 FMAs (~128 cycles).
template <int MODE>
__global__ __launch_bounds__(512, 1) void coexec_kernel(float* out, unsigned long long* cyc, float seed) {
  const int w = threadIdx.x >> 6;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (i + 1));
    b[i] = (__bf16)(seed - i);
  }
  f32x16 acc[4] = {};
  float x[32];
  for (int i = 0; i < 32; ++i) x[i] = seed + i + threadIdx.x;
  const float m = 0.999f, c = seed;
  const bool do_m = MODE == 0 || MODE == 3 || (MODE == 2 && w < 4);
  const bool do_v = MODE == 1 || MODE == 3 || (MODE == 2 && w >= 4);
  const unsigned long long t0 = clock64();
  for (int it = 0; it < CO_IT; ++it) {
    if (do_m && do_v) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[q], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[8 * q + i] = __builtin_fmaf(x[8 * q + i], m, c);
      }
    } else if (do_m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[q], 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = __builtin_fmaf(x[i], m, c);
    }
  }
  const unsigned long long t1 = clock64();
  float s = 0.f;
  for (int i = 0; i < 4; ++i) s += acc[i][threadIdx.x & 15];
  for (int i = 0; i < 32; ++i) s += x[i];
  out[blockIdx.x * 512 + threadIdx.x] = s;
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * 8 + w] = t1 - t0;
}

template <int MODE>
double coexec_cycles(int cus) {
  float* out;
  unsigned long long* cyc;
  CHECK(hipMalloc(&out, (size_t)cus * 512 * 4));
  CHECK(hipMalloc(&cyc, (size_t)cus * 8 * 8));
  hipLaunchKernelGGL(coexec_kernel<MODE>, dim3(cus), dim3(512), 0, 0, out, cyc, 0.5f);
  hipLaunchKernelGGL(coexec_kernel<MODE>, dim3(cus), dim3(512), 0, 0, out, cyc, 0.5f);
  CHECK(hipDeviceSynchronize());
  unsigned long long h[8];
  CHECK(hipMemcpy(h, cyc, 64, hipMemcpyDeviceToHost));
  unsigned long long mx = 0;
  for (int i = 0; i < 8; ++i) mx = h[i] > mx ? h[i] : mx;
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  return (double)mx / CO_IT;  // cycles per iteration of the slowest wave
}

int main() {
  int dev = 0, cus = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  double bf16_tf, bf16_cyc, fp8_tf, fp8_cyc, bf16r_tf, bf16r_cyc, fp8r_tf, fp8r_cyc, rd, cp;
  mfma_rate<0>(cus, bf16_tf, bf16_cyc);
  mfma_rate<1>(cus, fp8_tf, fp8_cyc);
  mfma_rate<2>(cus, bf16r_tf, bf16r_cyc);
  mfma_rate<3>(cus, fp8r_tf, fp8r_cyc);
  hbm(cus, rd, cp);
  const double lds128 = lds_bytes_per_clk<0>(cus), ldstr = lds_bytes_per_clk<1>(cus);
  const double fma_c = valu_cycles<0>(), exp_c = valu_cycles<1>();
  const double co0 = coexec_cycles<0>(cus), co1 = coexec_cycles<1>(cus), co2 = coexec_cycles<2>(cus),
               co3 = coexec_cycles<3>(cus);
  printf("{\"cus\": %d, \"mfma_bf16_tflops\": %.1f, \"mfma_bf16_cycles_per_inst\": %.2f, "
         "\"mfma_fp8_tflops\": %.1f, \"mfma_fp8_cycles_per_inst\": %.2f, \"hbm_read_gbs\": %.0f, "
         "\"hbm_copy_gbs\": %.0f, \"lds_b128_bytes_per_clk_cu\": %.1f, \"lds_tr_b16_bytes_per_clk_cu\": %.1f, "
         "\"valu_fma_cycles\": %.2f, \"valu_exp_cycles\": %.2f, \"coexec_cycles_mfma_only\": %.1f, "
         "\"coexec_cycles_valu_only\": %.1f, \"coexec_cycles_split_waves\": %.1f, "
         "\"coexec_cycles_interleaved\": %.1f, \"mfma_bf16_random_tflops\": %.1f, "
         "\"mfma_bf16_random_cycles_per_inst\": %.2f, \"mfma_fp8_random_tflops\": %.1f, "
         "\"mfma_fp8_random_cycles_per_inst\": %.2f}\n",
         cus, bf16_tf, bf16_cyc, fp8_tf, fp8_cyc, rd, cp, lds128, ldstr, fma_c, exp_c, co0, co1, co2, co3, bf16r_tf,
         bf16r_cyc, fp8r_tf, fp8r_cyc);
  return 0;
}
