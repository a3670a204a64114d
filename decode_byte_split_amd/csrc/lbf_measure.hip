// lbf_measure.hip — liblbf_measure.so: the read-stream ceiling that the
// benchmark reports the fused kernels against (measurement only; not part
// of the coded-weight path and not declared in include/lbf.h).
//
// Every byte of a device buffer is read once with 128-bit non-temporal loads,
// eight independent loads per lane in flight per iteration (one 256-thread
// workgroup per CU measured fastest), and XOR-reduced so that no load is
// dead; each workgroup stores its own XOR to its own word.  (One atomic per
// wave to a single word instead cost about 9 us a launch: 1024 atomics on one
// address serialise.)
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kUnroll = 8;  // loads in flight per lane (best of a sweep over 1-8 and 1-64 blocks per CU)

__global__ __launch_bounds__(256) void k_read_stream(const u32x4* __restrict__ p, uint64_t n16, uint32_t* out) {
  __shared__ uint32_t red[4];
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63u) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

extern "C" {

// Reads `bytes` bytes at d (16-byte aligned, bytes a multiple of 16) with
// `blocks` workgroups; d_out[b] (blocks words) receives the XOR of the
// 32-bit words workgroup b read.  Enqueued on s.
int lbfm_read_stream(const void* d, uint64_t bytes, uint32_t* d_out, int blocks, hipStream_t s) {
  if (!d || !d_out || (reinterpret_cast<uintptr_t>(d) & 15u) || (bytes & 15u) || blocks < 1) return -1;
  hipLaunchKernelGGL(k_read_stream, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<const u32x4*>(d),
                     bytes / 16, d_out);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
