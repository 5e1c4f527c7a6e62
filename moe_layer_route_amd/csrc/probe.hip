// Measurement probes: what the matrix cores and HBM of this GPU deliver to a
// plain hand-written kernel.  They are the "achievable" context printed next
// to the roofline fractions (which use the published peaks); they are not part
// of the MoE block.
//
// probe_mfma_kernel: every wave issues iters rounds of eight independent
//   v_mfma_f32_32x32x16_bf16 (eight accumulators spaced eight issues apart
//   hide the MFMA latency).  With all-ones operands every accumulator element
//   ends at 16 * iters, and lane 0's sum of its 128 elements at 2048 * iters,
//   both exact in float32 for iters <= 8191, so the output doubles as a check.
// probe_read_kernel: each workgroup streams one contiguous chunk of the buffer
//   with 16-byte loads, consecutive lanes on consecutive 16 bytes (whole
//   128-byte lines per eight lanes), eight loads (32 KB per workgroup) in
//   flight, XOR-folded and reduced to one word per wave.
//   Each 16-byte piece is read exactly once, so the XOR of all outputs equals
//   the XOR of the buffer's 32-bit words.
// probe_dot_kernel: the bf16 dot products of rows of A with rows of B as the
//   router forms them, v_mfma_f32_16x16x32_bf16 over K in steps of 32 into
//   one float32 accumulator, so that the MFMA's own accumulation error can be
//   measured against exact sums (bf16 x bf16 products are exact in float32;
//   what the instruction does with a step's 32 products and the accumulator
//   is not documented).  One wave per 16 rows of A.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kPbThreads = 256;
constexpr int kPbWaves = kPbThreads / kWave;
constexpr int kPbAcc = 8;
constexpr int kPbUnroll = 8;

__global__ __launch_bounds__(kPbThreads) void probe_mfma_kernel(int iters, float* __restrict__ out) {
  const u32x4_t one = u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // eight bf16 1.0
  f32x16_t acc[kPbAcc];
#pragma unroll
  for (int j = 0; j < kPbAcc; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kPbAcc; ++j) acc[j] = mfma32x32x16(one, one, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPbAcc; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  // lane 0 of each wave: 8 accumulators x 16 elements x 16 * iters
  if ((threadIdx.x & (kWave - 1)) == 0) out[blockIdx.x * kPbWaves + threadIdx.x / kWave] = s;
}

__global__ __launch_bounds__(kPbThreads) void probe_read_kernel(const u32x4_t* __restrict__ buf, size_t n16,
                                                                 size_t chunk16, uint32_t* __restrict__ out) {
  // workgroup b reads pieces [b chunk16, (b + 1) chunk16) of the buffer
  const size_t begin = (size_t)blockIdx.x * chunk16;
  const size_t end = min(begin + chunk16, n16);
  size_t i = begin + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kPbUnroll - 1) * kPbThreads < end; i += kPbUnroll * kPbThreads) {
    u32x4_t v[kPbUnroll];
#pragma unroll
    for (int u = 0; u < kPbUnroll; ++u) v[u] = ld16(buf + i + u * kPbThreads);
#pragma unroll
    for (int u = 0; u < kPbUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kPbThreads) {
    const u32x4_t v = ld16(buf + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) x ^= (uint32_t)__shfl_xor((int)x, d, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) out[blockIdx.x * kPbWaves + threadIdx.x / kWave] = x;
}

__global__ __launch_bounds__(kWave) void probe_dot_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ B,
                                                           int K, float* __restrict__ out) {
  // lane l: A row 16 b + l%16 and B row l%16, K chunk 8 (l/16) of every step
  const int lane = threadIdx.x;
  const int c = lane & 15, g = lane >> 4;
  const bf16_t* a = A + ((size_t)blockIdx.x * 16 + c) * K + 8 * g;
  const bf16_t* b = B + (size_t)c * K + 8 * g;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += 32) acc = mfma16x16x32(ld16(a + k0), ld16(b + k0), acc);
  // accumulator layout: lane l, element v = A row 4 (l/16) + v, B row l%16
#pragma unroll
  for (int v = 0; v < 4; ++v) out[((size_t)blockIdx.x * 16 + 4 * g + v) * 16 + c] = acc[v];
}

}  // namespace

hipError_t launch_probe_dot(const void* A, const void* B, int M, int K, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(probe_dot_kernel, dim3((unsigned)(M / 16)), dim3(kWave), 0, stream, (const bf16_t*)A,
                     (const bf16_t*)B, K, out);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, int workgroups, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)workgroups), dim3(kPbThreads), 0, stream, iters, out);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* buf, size_t bytes, int workgroups, uint32_t* out, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t chunk16 = ((n16 + workgroups - 1) / workgroups + kPbThreads - 1) / kPbThreads * kPbThreads;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)workgroups), dim3(kPbThreads), 0, stream,
                     (const u32x4_t*)buf, n16, chunk16, out);
  return hipGetLastError();
}

}  // namespace moe
