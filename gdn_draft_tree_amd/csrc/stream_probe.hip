// Streaming probe for the benchmark (not part of the verification path): plain kernels that
// move a given number of bytes with no arithmetic, to measure what this part streams for a
// given traffic mix.  Built into its own library, libgdntree_probe.so, so the path's C ABI
// stays as declared in gdntree.h.
//
// gdntree_probe_stream: `blocks` workgroups of 256 threads; workgroup u reads its contiguous
// share of `read_bytes` from `src` (16-byte loads, consecutive lanes on consecutive chunks,
// four loads in flight per lane) and then writes its contiguous share of `write_bytes` to
// `dst`.  A value folded from the reads decides nothing the host can see but keeps the loads
// alive.  With blocks = the verify launch's units and its per-unit read and write sizes, this
// is the verify kernel's traffic with none of its work.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_kernel(const u32x4 *__restrict__ src, size_t rchunks_per_block,
                                                     size_t rchunks, u32x4 *__restrict__ dst,
                                                     size_t wchunks_per_block, size_t wchunks) {
  const size_t u = blockIdx.x;
  const size_t r0 = u * rchunks_per_block;
  const size_t r1 = r0 + rchunks_per_block < rchunks ? r0 + rchunks_per_block : rchunks;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = r0 + threadIdx.x;
  for (; i + 3 * 256 < r1; i += 4 * 256) {
    const u32x4 a = __builtin_nontemporal_load(src + i), b = __builtin_nontemporal_load(src + i + 256);
    const u32x4 c = __builtin_nontemporal_load(src + i + 512), d = __builtin_nontemporal_load(src + i + 768);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < r1; i += 256) acc ^= __builtin_nontemporal_load(src + i);
  const size_t w0 = u * wchunks_per_block;
  const size_t w1 = w0 + wchunks_per_block < wchunks ? w0 + wchunks_per_block : wchunks;
  // the folded value is all-ones only if the reads were; the writes carry zero otherwise
  const unsigned keep = (acc.x & acc.y & acc.z & acc.w) == 0xffffffffu ? 1u : 0u;
  for (size_t j = w0 + threadIdx.x; j < w1; j += 256) dst[j] = u32x4{keep, 0u, 0u, 0u};
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int gdntree_probe_stream(const void *src, size_t read_bytes,
                                                                          void *dst, size_t write_bytes,
                                                                          int blocks, hipStream_t stream) {
  if (blocks <= 0 || (read_bytes && !src) || (write_bytes && !dst) || read_bytes % 16 || write_bytes % 16) return 1;
  const size_t rch = read_bytes / 16, wch = write_bytes / 16;
  const size_t rpb = (rch + blocks - 1) / blocks, wpb = (wch + blocks - 1) / blocks;
  hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const u32x4 *>(src),
                     rpb, rch, static_cast<u32x4 *>(dst), wpb, wch);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}
