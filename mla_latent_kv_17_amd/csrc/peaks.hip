// Measurement probes (not part of the decode library): the HBM read rate and
// the bf16 matrix-core rate this part reaches in practice, reported by the
// benchmark next to the published peaks.  Built into its own library,
// libmla_peaks.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"

namespace {

using namespace mla;

// Streaming read: block b reads its own contiguous 1/gridDim share of the
// buffer, each thread eight 16-byte loads in flight per trip (32 KB per block
// per trip), folded into one word so the loads stay live; one word per
// thread goes to `sink`.
__global__ void __launch_bounds__(256) probe_read(const u32x4* buf, int64_t n16, uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = i + k * 256 < hi ? buf[i + k * 256] : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Eight independent 32x32x16 bf16 products per trip on each wave's own
// accumulators, `iters` trips; the sums go to `sink` so nothing is dropped.
__global__ void __launch_bounds__(256) probe_mfma(float* sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a = as_bf16x8(u32x4{0x3F803F80u + lane, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  bf16x8 b = as_bf16x8(u32x4{0x3C003C00u, 0x3C003C00u + lane, 0x3C003C00u, 0x3C003C00u});
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = mfma32x32x16(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[k][j];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// sink: at least blocks * 256 words.  Returns 0, or the HIP error code.
int mla_probe_read(const void* buf, int64_t bytes, uint32_t* sink, int blocks, void* stream) {
  hipLaunchKernelGGL(probe_read, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf, bytes / 16, sink);
  return (int)hipGetLastError();
}

// flops of one call: blocks * 4 waves * iters * 8 * 2 * 32 * 32 * 16
int mla_probe_mfma(float* sink, int blocks, int iters, void* stream) {
  hipLaunchKernelGGL(probe_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, sink, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
