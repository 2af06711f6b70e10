// Plain streaming read (a measurement aid, not a step of the linear): every
// byte of a buffer is loaded once with 16-byte loads, each thread keeping
// kStreamU loads in flight, and folded into an XOR per workgroup; workgroup b
// stores its XOR to sink[b] (a few kilobytes in all, so the loads cannot be
// dropped and the writes do not count).  Its rate is the HBM read rate the
// weight-streaming kernels can be held against (loaded with the nontemporal
// hint, as they load their weights).
#include "device_common.hpp"
#include "launch.hpp"

namespace nvfp4 {

namespace {

constexpr int kStreamU = 8;
constexpr int kStreamThreads = 256;

__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const uint4* __restrict__ src, int64_t n_vec,
                                                                     uint32_t* __restrict__ sink) {
  __shared__ uint32_t part[kStreamThreads / 64];
  uint32_t x = 0;
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads * kStreamU;
  for (int64_t i0 = (int64_t)blockIdx.x * kStreamThreads * kStreamU + threadIdx.x; i0 < n_vec; i0 += stride) {
    uint4 v[kStreamU];
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const int64_t i = i0 + (int64_t)u * kStreamThreads;
      v[u] = ld_stream16(src + (i < n_vec ? i : n_vec - 1));  // past the end: an in-bounds load, value dropped below
    }
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) {
      const uint32_t f = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      x ^= i0 + (int64_t)u * kStreamThreads < n_vec ? f : 0u;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kStreamThreads / 64; ++w) t ^= part[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

int64_t stream_read_blocks(int64_t bytes) {
  const int64_t n_vec = bytes / 16;
  const int64_t blocks = (n_vec + kStreamThreads * kStreamU - 1) / (kStreamThreads * kStreamU);
  return blocks > kStreamSinkWords ? kStreamSinkWords : (blocks < 1 ? 1 : blocks);
}

void launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  stream_read_kernel<<<(unsigned)stream_read_blocks(bytes), kStreamThreads, 0, s>>>(static_cast<const uint4*>(src),
                                                                                   bytes / 16, sink);
}

}  // namespace nvfp4
