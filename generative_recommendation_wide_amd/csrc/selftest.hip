// Device self-check of the wave primitives in device_common.h: each register lane exchange,
// scan and reduction against the general shuffle form (ds_bpermute) that it replaces.
#include "device_common.h"
#include "grw_internal.h"

using namespace grw;

namespace {

constexpr int kChecks = 14;

__device__ uint32_t shfl_xor_ref(uint32_t x, int o) { return __shfl_xor(x, o, 64); }

__device__ int scan_ref(int v) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ uint32_t max_scan_ref(uint32_t v) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v = max(v, t);
  }
  return v;
}

template <typename T>
__device__ T sum_ref(T v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ T max_ref(T v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// One workgroup of 256 threads; check c of thread t writes out[c * 256 + t] = 1 when the two
// forms agree (bit for bit), else 0.
__global__ __launch_bounds__(256) void lanes_selftest_kernel(int32_t* out) {
  const int t = threadIdx.x, lane = t & 63;
  const uint32_t x = (0x9E3779B9u * (uint32_t)(t + 1)) ^ ((uint32_t)t << 7);
  int c = 0;
  out[c++ * 256 + t] = lane_xor<1>(x) == shfl_xor_ref(x, 1);
  out[c++ * 256 + t] = lane_xor<2>(x) == shfl_xor_ref(x, 2);
  out[c++ * 256 + t] = lane_xor<4>(x) == shfl_xor_ref(x, 4);
  out[c++ * 256 + t] = lane_xor<8>(x) == shfl_xor_ref(x, 8);
  out[c++ * 256 + t] = lane_xor<16>(x) == shfl_xor_ref(x, 16);
  out[c++ * 256 + t] = lane_xor<32>(x) == shfl_xor_ref(x, 32);
  const uint64_t u = ((uint64_t)x << 32) | (uint64_t)(x * 7u + 3u);
  out[c++ * 256 + t] = lane_xor<4>(u) == (((uint64_t)shfl_xor_ref((uint32_t)(u >> 32), 4) << 32) |
                                          shfl_xor_ref((uint32_t)u, 4));
  const uint32_t before = __shfl_up(x, 1, 64);
  out[c++ * 256 + t] = lane_before(x) == (lane ? before : 0u);
  const int v = (int)(x & 0xffu);
  out[c++ * 256 + t] = wave_inclusive_scan(v) == scan_ref(v);
  out[c++ * 256 + t] = wave_inclusive_max_scan(x >> 4) == max_scan_ref(x >> 4);
  const double d = (double)x * 1.2345e-7 - 17.0 / (double)(t + 3);
  out[c++ * 256 + t] = __double_as_longlong(wave_sum(d)) == __double_as_longlong(sum_ref(d));
  const float f = (float)d * ((t & 1) ? -1.0f : 1.0f);
  out[c++ * 256 + t] = __float_as_uint(wave_sum(f)) == __float_as_uint(sum_ref(f));
  out[c++ * 256 + t] = __float_as_uint(wave_max(f)) == __float_as_uint(max_ref(f));
  out[c++ * 256 + t] = wave_max(x) == max_ref(x);
}

static_assert(kChecks * 256 == GRW_SELFTEST_WORDS, "one word per check and thread");

}  // namespace

extern "C" int grw_selftest_lanes(int32_t* scratch, void* stream, int32_t* mismatches) {
  if (scratch == nullptr || mismatches == nullptr) return GRW_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  lanes_selftest_kernel<<<1, 256, 0, s>>>(scratch);
  if (hipGetLastError() != hipSuccess) return GRW_EDEVICE;
  int32_t h[GRW_SELFTEST_WORDS];
  if (hipMemcpyAsync(h, scratch, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return GRW_EDEVICE;
  int32_t bad = 0;
  for (int i = 0; i < GRW_SELFTEST_WORDS; ++i) bad += h[i] != 1;
  *mismatches = bad;
  return GRW_OK;
}
