// Read-bandwidth probe for the schedule choice.
//
// "Kernel optimization for MiniMax M3 on NVIDIA Blackwell" (section 1 and the appendix): the
// KV-outer / Q-outer crossover follows from the ratio of cache to HBM bandwidth, measured on
// the machine. The probe sweeps the first `working_set` bytes of a buffer again and again
// until `total` bytes have been read: every sweep is one coalesced pass of the whole grid
// (workgroup b reads the 4 KiB pieces b, b + grid, ...), so a working set larger than the
// last-level cache streams from HBM and a smaller one is served from the cache. Each thread
// folds what it read into a sum that it writes out, so no load can be elided.
#include "msa_device.h"
#include "msa_internal.h"

namespace msa {
namespace {

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ buf,
                                                         uint64_t n_pieces, uint64_t n_iter,
                                                         float* __restrict__ sink) {
  // a piece is 4 KiB: 256 threads x 16 bytes
  const uint64_t grid = gridDim.x;
  uint64_t piece = blockIdx.x;
  uint32_t acc = 0;
  for (uint64_t it = 0; it < n_iter; ++it) {
    const u32x4 v = buf[piece * 256 + threadIdx.x];
    acc += v[0] ^ v[1] ^ v[2] ^ v[3];
    piece += grid;
    if (piece >= n_pieces) piece -= n_pieces;
  }
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = (float)acc;
}

}  // namespace

hipError_t launch_probe_read(const void* buf, size_t working_set, size_t total, float* sink,
                             hipStream_t st) {
  const uint64_t n_pieces = working_set / 4096;
  const uint64_t n_iter = total / 4096 / kProbeGrid;
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeGrid), dim3(256), 0, st,
                     reinterpret_cast<const u32x4*>(buf), n_pieces, n_iter, sink);
  return hipGetLastError();
}

}  // namespace msa
