// Read-bandwidth probe: a plain streaming read of a device buffer, the
// reference a streaming kernel on this chip can reach, reported beside the
// rooflines' 8 TB/s.  Every 16-byte piece is read once: each workgroup
// streams one contiguous slice, its 256 threads reading consecutive pieces,
// eight pieces in flight per thread (contiguous slices measured 6.3 TB/s
// against 5.8 TB/s for a grid-stride walk at the same depth).  The pieces are
// folded by XOR into one 32-bit word per workgroup, so no read can be dropped
// and the result is checkable.  No atomics: each workgroup writes its own
// word.
#include "internal.h"

using namespace medusa;

namespace {

constexpr int PT = 256;       // threads per workgroup
constexpr int PGRID = 8192;   // workgroups (32 per CU of a 256-CU chip)
constexpr int PUNROLL = 8;    // 16-byte pieces in flight per thread

__global__ __launch_bounds__(PT) void read_probe_kernel(const uint4* p, int64_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;  // pieces of this workgroup's slice
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
  int64_t i = b0 + threadIdx.x;
  for (; i + (PUNROLL - 1) * PT < b1; i += PUNROLL * PT) {
    uint4 v[PUNROLL];
#pragma unroll
    for (int u = 0; u < PUNROLL; ++u) v[u] = p[i + u * PT];
#pragma unroll
    for (int u = 0; u < PUNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += PT) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off, 64));
  __shared__ uint32_t s[PT / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

}  // namespace

extern "C" int medusa_read_probe_partials(void) { return PGRID; }

extern "C" int medusa_read_probe(const void* buf, size_t bytes, uint32_t* partials, hipStream_t stream) {
  clear_error();
  MEDUSA_CHECK_ARG((buf || bytes == 0) && partials, "buf (unless bytes is 0) and partials must be non-NULL");
  MEDUSA_CHECK_ARG(bytes % 16 == 0 && aligned16(buf), "the buffer must be 16-byte aligned and a multiple of 16 bytes");
  hipLaunchKernelGGL(read_probe_kernel, dim3(PGRID), dim3(PT), 0, stream, static_cast<const uint4*>(buf),
                     static_cast<int64_t>(bytes / 16), partials);
  return check_launch("read probe");
}
