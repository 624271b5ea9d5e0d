// Streaming-read probe for bench.py (measurement only; not part of
// libdiffattn.so): the HBM read rate a plain, well-formed read kernel reaches on
// this device, the measured reference printed next to the published 8 TB/s on
// the bandwidth-bound decode lines.  Every thread reads 16-byte vectors with
// non-temporal loads (the data is read once), four in flight per iteration,
// over a grid-stride range of 16384 workgroups; the values are folded into one
// word that is stored only if it equals an unlikely constant, so the loads
// cannot be dropped and the kernel writes (practically) nothing.
//
// C entry point (built into bench_probe.so next to this file):
//   int bench_hbm_read_probe(const void* src, size_t nbytes, float* sink, void* stream)
// src: device, 16-byte aligned, nbytes a multiple of 16 (0 = no-op); sink:
// device fp32 [1], 4-byte aligned, not inside src.  Returns 0 on success, 1 on
// invalid arguments (nothing launched), 3 on a launch failure.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 256;
constexpr int kBlocks = 16384;  // 64 workgroups per CU on 256 CUs

__global__ __launch_bounds__(kT) void hbm_read_probe_kernel(const u32x4* __restrict__ src, int64_t n16, float* sink) {
  const int64_t stride = (int64_t)gridDim.x * kT;
  int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(&src[i]), b = __builtin_nontemporal_load(&src[i + stride]);
    const u32x4 c = __builtin_nontemporal_load(&src[i + 2 * stride]), d = __builtin_nontemporal_load(&src[i + 3 * stride]);
    acc ^= (a[0] ^ a[1] ^ a[2] ^ a[3]) + (b[0] ^ b[1] ^ b[2] ^ b[3]) + (c[0] ^ c[1] ^ c[2] ^ c[3]) +
           (d[0] ^ d[1] ^ d[2] ^ d[3]);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = src[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = 1.0f;
}

}  // namespace

extern "C" int bench_hbm_read_probe(const void* src, size_t nbytes, float* sink, void* stream) {
  if (nbytes == 0) return 0;
  if (!src || !sink) return 1;
  if ((uintptr_t)src % 16 != 0 || nbytes % 16 != 0 || (uintptr_t)sink % 4 != 0) return 1;
  if (nbytes > ((size_t)1 << 40)) return 1;
  const uintptr_t s0 = (uintptr_t)sink, lo = (uintptr_t)src;
  if (s0 + sizeof(float) > lo && s0 < lo + nbytes) return 1;
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(kBlocks), dim3(kT), 0, (hipStream_t)stream, (const u32x4*)src,
                     (int64_t)(nbytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
