// Measurement probe, not part of the forward: reads a (B, T, H, 16) bf16 tensor the way the chunked
// read-out kernel reads its q and k rows (one workgroup per (b, h); a wave loads 32 tokens' 32-byte rows
// with 16-byte loads, two lanes per row, at a stride of H * 32 bytes; blocks dealt to the 8 XCDs round
// robin with the (b, h) pairs in contiguous runs per XCD, so that the heads sharing a 128-byte line meet
// in one L2). Every byte of the tensor is read exactly once per launch, which makes the bytes a profiler
// counter should report known. The values are folded into one word per thread so the loads are kept.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(64) void probe_read_rows_kernel(const uint4* __restrict__ x, int64_t T, int64_t H,
                                                              int64_t pairs, unsigned* __restrict__ sink) {
  const int64_t ppx = pairs / 8;
  const int64_t pair = (blockIdx.x & 7) * ppx + (blockIdx.x >> 3);  // XCD x % 8 takes the x-th run of pairs
  const int64_t b = pair / H, h = pair % H;
  const int lane = threadIdx.x;
  const uint4* base = x + ((b * T) * H + h) * 2;  // 16 bf16 = two 16-byte units per row
  unsigned acc = 0;
  for (int64_t t0 = 0; t0 < T; t0 += 32) {
    const int64_t t = t0 + lane / 2;
    if (t < T) {
      const uint4 u = base[t * H * 2 + (lane & 1)];
      acc ^= u.x ^ u.y ^ u.z ^ u.w;
    }
  }
  sink[pair * 64 + lane] = acc;
}

}  // namespace

// x: (B, T, H, 16) bf16 device tensor; sink: B * H * 64 unsigned words. Returns 0, 1 for bad arguments
// (B * H must be a multiple of 8), 2 when the launch fails.
extern "C" int based_probe_read_rows(const void* x, int64_t B, int64_t T, int64_t H, unsigned* sink,
                                     hipStream_t stream) {
  const int64_t pairs = B * H;
  if (!x || !sink || B < 1 || T < 1 || H < 1 || pairs % 8 != 0 || pairs > (int64_t(1) << 30)) return 1;
  hipLaunchKernelGGL(probe_read_rows_kernel, dim3(static_cast<unsigned>(pairs)), dim3(64), 0, stream,
                     static_cast<const uint4*>(x), T, H, pairs, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
