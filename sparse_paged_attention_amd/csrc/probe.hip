// Read-bandwidth probe: the memory-access shape of the attention's page reads
// (whole 4 KiB pieces at scattered places in a large buffer, each read once),
// with no arithmetic behind it. The benchmark times it on the same GPU to give
// the attention kernel a measured ceiling next to the HBM peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spa_probe.h"

namespace {

// One 64-lane wave reads CPW chunks of 4 KiB, every load issued before the
// first is used (lane l reads 16 bytes at l, l + 64, l + 128 and l + 192 of
// each chunk: four 1 KiB coalesced loads per chunk), and folds what it read
// into one word so that nothing is optimised away.
template <int CPW>
__global__ void __launch_bounds__(64) read_probe_kernel(const uint4* __restrict__ base,
                                                        const int32_t* __restrict__ ids, int32_t n,
                                                        uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  const int32_t c0 = (int32_t)blockIdx.x * CPW;
  uint4 v[CPW][4];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int32_t id = ids[min(c0 + u, n - 1)];
    const uint4* p = base + (int64_t)id * 256 + lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[u][i] = p[64 * i];
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < CPW; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc ^= v[u][i].x ^ v[u][i].y ^ v[u][i].z ^ v[u][i].w;
#pragma unroll
  for (int o = 32; o; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (lane == 0) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int spa_probe_read_chunks(const void* base, size_t base_bytes, const int32_t* chunk_ids,
                                     int32_t n_chunks, int32_t chunks_per_wave, uint32_t* sink,
                                     hipStream_t stream) {
  if (!base || !chunk_ids || !sink || n_chunks < 1 || base_bytes < 4096) return 1;
  const int32_t waves = (n_chunks + chunks_per_wave - 1) / chunks_per_wave;
  const uint4* b = static_cast<const uint4*>(base);
  switch (chunks_per_wave) {
    case 4: hipLaunchKernelGGL(read_probe_kernel<4>, dim3(waves), dim3(64), 0, stream, b, chunk_ids, n_chunks, sink); break;
    case 8: hipLaunchKernelGGL(read_probe_kernel<8>, dim3(waves), dim3(64), 0, stream, b, chunk_ids, n_chunks, sink); break;
    case 16: hipLaunchKernelGGL(read_probe_kernel<16>, dim3(waves), dim3(64), 0, stream, b, chunk_ids, n_chunks, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
