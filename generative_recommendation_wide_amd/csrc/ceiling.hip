// Measurement kernel for the benchmark's achievable ceilings; not part of the decode path and
// built into its own library (libgrw_ceiling.so).  It measures the dense bf16 MFMA rate of the
// whole chip under sustained load and the shader clock the chip runs at meanwhile, the two
// figures that set how far any MFMA-bound kernel can get below the spec peak (which assumes
// the 2.4 GHz peak engine clock).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kAcc = 8;             // independent accumulations per wave
constexpr int kLdsHold = 96 * 1024; // dynamic LDS each workgroup holds (unused): with 160 KB per
                                    // CU, no two workgroups share a CU

// One 4-wave workgroup per CU (one wave per SIMD; the LDS each workgroup reserves keeps a
// second one off its CU, so no CU runs two while another idles).  Each wave keeps kAcc independent
// v_mfma_f32_32x32x16_bf16 accumulations in flight, so the matrix pipe of its SIMD never waits
// on a result; operands are fixed registers, so no memory traffic competes.  Thread 0 records
// the workgroup's shader-clock cycles (s_memtime) and 100 MHz wall-clock ticks (s_memrealtime)
// across the loop.
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* out, uint64_t* ts) {
  bf16x8 a[kAcc], b[kAcc];
  uint32_t h = threadIdx.x * 2654435761u + blockIdx.x * 40503u;
  for (int j = 0; j < kAcc; ++j)
    for (int i = 0; i < 8; ++i) {
      h = h * 1664525u + 1013904223u;
      a[j][i] = (__bf16)((float)((h >> 9) & 1023) * (1.0f / 1024.0f) - 0.5f);
      h = h * 1664525u + 1013904223u;
      b[j][i] = (__bf16)((float)((h >> 9) & 1023) * (1.0f / 1024.0f) - 0.5f);
    }
  floatx16 c[kAcc];
  for (int j = 0; j < kAcc; ++j) c[j] = floatx16{};
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], c[j], 0, 0, 0);
  }
  float s = 0.0f;
  for (int j = 0; j < kAcc; ++j)
    for (int e = 0; e < 16; ++e) s += c[j][e];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    ts[blockIdx.x * 4] = t1 - t0;
    ts[blockIdx.x * 4 + 1] = r1 - r0;
    ts[blockIdx.x * 4 + 2] = r0;
    ts[blockIdx.x * 4 + 3] = r1;
  }
}

}  // namespace

extern "C" {

// Launch `blocks` workgroups of the MFMA rate kernel, each running `iters` rounds of
// 8 MFMAs per wave (4 waves, 32768 flops per MFMA).  out: device float[blocks * 256]
// (results kept live); ts: device uint64[blocks * 4], per workgroup the shader cycles and the
// 100 MHz ticks of its loop, and the 100 MHz clock at its start and end.  Returns 0, -1 on invalid arguments, -2 on a launch error.
int grw_ceiling_mfma(int32_t blocks, int32_t iters, float* out, uint64_t* ts, void* stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr || ts == nullptr) return -1;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)mfma_rate_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsHold) !=
        hipSuccess)
      return -2;
    attr_set = true;
  }
  mfma_rate_kernel<<<blocks, 256, kLdsHold, (hipStream_t)stream>>>(iters, out, ts);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

int grw_ceiling_mfma_per_round(void) { return kAcc; }

}  // extern "C"
