// Measurement probes: what this chip actually sustains, for the roofline
// denominators beside the published peaks.
//
//   * HBM streams over caller buffers far larger than the last-level cache:
//     a copy (every byte read once and written once), a read-only pass (a
//     sum per thread, one store per thread at the end) and a write-only fill.
//     16-byte vector accesses, a grid of 8 workgroups per compute unit
//     striding over the buffer, eight accesses per thread and pass with every
//     load issued before the first store (one access per pass leaves too few
//     bytes in flight: on 2 GiB buffers the copy then ran 4.7 TB/s against
//     5.3, the fill 4.5 against 5.6; streaming or plain stores made no
//     difference at eight per pass).
//   * The matrix-core rate: every wave issues back-to-back
//     v_mfma_f32_32x32x16_bf16 into four independent accumulators (so no
//     product waits on the previous one), 8 waves per compute unit, one
//     workgroup per compute unit; the accumulators are written out at the end
//     so nothing is removed by the compiler.
// Each probe launches `iters` times between two HIP events on `stream` after
// one untimed warm-up launch and reports the mean time per launch.

#include "kvx_internal.hpp"

namespace kvx {

constexpr int PH_U = 8;  // 16-byte accesses per thread and pass, 256 apart

__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * PH_U;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 * PH_U + threadIdx.x; i0 < n16; i0 += stride) {
    u32x4 v[PH_U];
#pragma unroll
    for (int k = 0; k < PH_U; ++k) {
      const int64_t i = i0 + k * 256;
      v[k] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < PH_U; ++k) {
      const int64_t i = i0 + k * 256;
      if (i < n16) dst[i] = v[k];
    }
  }
}

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ sink,
                                                         int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * PH_U;
  uint32_t acc = 0;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 * PH_U + threadIdx.x; i0 < n16; i0 += stride) {
    u32x4 v[PH_U];
#pragma unroll
    for (int k = 0; k < PH_U; ++k) {
      const int64_t i = i0 + k * 256;
      v[k] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < PH_U; ++k) acc += v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = acc;
}

__global__ __launch_bounds__(256) void probe_fill_kernel(u32x4* __restrict__ dst, int64_t n16, uint32_t v) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * PH_U;
  for (int64_t i0 = static_cast<int64_t>(blockIdx.x) * 256 * PH_U + threadIdx.x; i0 < n16; i0 += stride) {
#pragma unroll
    for (int k = 0; k < PH_U; ++k) {
      const int64_t i = i0 + k * 256;
      if (i < n16) dst[i] = u32x4{v, v, v, v};
    }
  }
}

constexpr int PM_CHAIN = 4;  // independent accumulators per wave
__global__ __launch_bounds__(512) void probe_mfma_kernel(float* __restrict__ out, int32_t reps, uint32_t seed) {
  const int lane = threadIdx.x & 63;
  // operands: small bf16 values from the lane and seed, so the sums stay finite
  const uint32_t h = (seed ^ (lane * 0x9e3779b9u)) & 0x007f007fu;
  const u32x4 a = u32x4{0x3f803f80u ^ h, 0x3f803f80u, 0x3f803f80u ^ (h >> 1), 0x3f803f80u};
  const u32x4 b = u32x4{0x3c003c00u, 0x3c003c00u ^ h, 0x3c003c00u, 0x3c003c00u ^ (h >> 2)};
  f32x16 acc[PM_CHAIN];
#pragma unroll
  for (int c = 0; c < PM_CHAIN; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  for (int32_t r = 0; r < reps; ++r) {
#pragma unroll
    for (int c = 0; c < PM_CHAIN; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                      acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < PM_CHAIN; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// Runs `launch` once untimed, then `iters` times between two events; mean ms.
template <typename F>
static int timed_launches(hipStream_t s, int32_t iters, float* ms, F&& launch) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return KVX_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return KVX_ERR_HIP;
  }
  int st = launch();
  if (st == KVX_OK && hipEventRecord(e0, s) != hipSuccess) st = KVX_ERR_HIP;
  for (int32_t i = 0; st == KVX_OK && i < iters; ++i) st = launch();
  if (st == KVX_OK && hipEventRecord(e1, s) != hipSuccess) st = KVX_ERR_HIP;
  if (st == KVX_OK && hipEventSynchronize(e1) != hipSuccess) st = KVX_ERR_HIP;
  float t = 0.0f;
  if (st == KVX_OK && hipEventElapsedTime(&t, e0, e1) != hipSuccess) st = KVX_ERR_HIP;
  if (st == KVX_OK) *ms = t / static_cast<float>(iters);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return st;
}

int run_probe_hbm(int32_t mode, void* a, void* b, int64_t bytes, int32_t iters, float* ms, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const unsigned grid = static_cast<unsigned>(device_cu_count() * 8);
  return timed_launches(s, iters, ms, [&]() -> int {
    if (mode == 0)
      probe_copy_kernel<<<grid, 256, 0, s>>>(static_cast<const u32x4*>(a), static_cast<u32x4*>(b), n16);
    else if (mode == 1)
      probe_read_kernel<<<grid, 256, 0, s>>>(static_cast<const u32x4*>(a), static_cast<uint32_t*>(b), n16);
    else
      probe_fill_kernel<<<grid, 256, 0, s>>>(static_cast<u32x4*>(a), n16, 0x3c003c00u);
    KVX_LAUNCH_CHECK();
    return KVX_OK;
  });
}

int run_probe_mfma(float* out, int32_t reps, int32_t iters, float* ms, double* flops, hipStream_t s) {
  const int cus = device_cu_count();
  *flops = static_cast<double>(cus) * 8 * PM_CHAIN * static_cast<double>(reps) * (2.0 * 32 * 32 * 16);
  return timed_launches(s, iters, ms, [&]() -> int {
    probe_mfma_kernel<<<static_cast<unsigned>(cus), 512, 0, s>>>(out, reps, 0x1234u);
    KVX_LAUNCH_CHECK();
    return KVX_OK;
  });
}

int probe_mfma_out_floats() { return device_cu_count() * 512; }
int probe_read_sink_words() { return device_cu_count() * 8 * 256; }

}  // namespace kvx
