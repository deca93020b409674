// hbm_read_probe.hip -- what a kernel with no computation reads from HBM.
//
// A memory-bound attention kernel (the decode forward streams K and V once)
// is priced against the published HBM3E peak; this stand-alone program gives
// the rate the same chip reaches with nothing but loads, as context for that
// fraction.  Each thread reads 16-byte words grid-stride over a 2 GiB buffer
// (four loads in flight per iteration), folds them with xor and writes one
// word, so every byte of the buffer is read once per launch.
//
//     io_aware_exact_fwd_amd/hbm_read_probe     (prints one line per launch shape)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NONTEMPORAL>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NONTEMPORAL) return __builtin_nontemporal_load(p);
  return *p;
}

// n16 words at a; out holds gridDim.x * 256 words.
template <bool NONTEMPORAL>
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ a, size_t n16,
                                                   unsigned* __restrict__ out) {
  size_t i = blockIdx.x * (size_t)256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 x0 = load16<NONTEMPORAL>(a + i), x1 = load16<NONTEMPORAL>(a + i + stride);
    const u32x4 x2 = load16<NONTEMPORAL>(a + i + 2 * stride), x3 = load16<NONTEMPORAL>(a + i + 3 * stride);
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  for (; i < n16; i += stride) acc ^= load16<NONTEMPORAL>(a + i);
  out[blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

}  // namespace

int main() {
  const size_t bytes = size_t(2) << 30;
  const size_t n16 = bytes / 16;
  const int grids[] = {1024, 2048, 4096, 8192, 16384};
  const int max_grid = 16384;
  u32x4* a = nullptr;
  unsigned* out = nullptr;
  hipEvent_t e0, e1;
  if (!ok(hipMalloc(&a, bytes), "hipMalloc") ||
      !ok(hipMalloc(&out, size_t(max_grid) * 256 * sizeof(unsigned)), "hipMalloc") ||
      !ok(hipMemset(a, 1, bytes), "hipMemset") || !ok(hipEventCreate(&e0), "hipEventCreate") ||
      !ok(hipEventCreate(&e1), "hipEventCreate"))
    return 1;
  double best = 0.0;
  for (int nt = 1; nt >= 0; --nt)
    for (int grid : grids) {
      auto kern = nt ? read_kernel<true> : read_kernel<false>;
      for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, 0, a, n16, out);
      const int reps = 20;
      if (!ok(hipEventRecord(e0), "hipEventRecord")) return 1;
      for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, 0, a, n16, out);
      if (!ok(hipEventRecord(e1), "hipEventRecord") || !ok(hipEventSynchronize(e1), "hipEventSynchronize"))
        return 1;
      float ms = 0.f;
      if (!ok(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime")) return 1;
      ms /= reps;
      const double gbps = bytes / (ms * 1e-3) / 1e9;
      if (gbps > best) best = gbps;
      std::printf("%s loads, %5d workgroups x 256: %8.1f us per 2 GiB read = %7.1f GB/s\n",
                  nt ? "non-temporal" : "plain       ", grid, ms * 1e3, gbps);
      std::fflush(stdout);
    }
  std::printf("best: %.1f GB/s (%.1f %% of 8000 GB/s)\n", best, best / 80.0);
  return ok(hipGetLastError(), "launch") && ok(hipDeviceSynchronize(), "sync") ? 0 : 1;
}
