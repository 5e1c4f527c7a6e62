// Routing-weighted combine of the k expert outputs of each token.
//
// xserv "Phase 19: gpt-oss-20b MoE support", section 2: the weighted sum takes
// only the top-k experts of each token; experts a token did not select are
// skipped (never multiplied by 0), so only the k selected rows of o are read.
// The sum runs in float32 in the fixed order j = 0..k-1 and is rounded once to
// bf16, so the result does not depend on launch order.  A slot with pos < 0
// (an expert another rank holds) is left out; the expert-parallel partial
// output is written in float32 instead, for the sum over ranks.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;

// KMAX >= k slots per token; every load of a thread is issued before the
// first product (slots past k re-read slot 0 and are left out of the sum).
// OUT_F32: float32 output (expert-parallel partial sums), else bf16.
template <int KMAX, bool OUT_F32>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ o, const int32_t* __restrict__ pos, const float* __restrict__ w,
    int64_t T, int H, int k, void* __restrict__ y) {
  // one thread per 4 consecutive columns of one token
  const int64_t item = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  const int quads = H / 4;
  if (item >= T * quads) return;   // no barrier in this kernel
  const int64_t t = item / quads;
  const int n = 4 * (int)(item - t * quads);
  int p[KMAX];
  float wj[KMAX];
  bool use[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const size_t s = (size_t)t * k + (j < k ? j : 0);
    const int ps = pos[s];
    use[j] = j < k && ps >= 0;
    p[j] = ps >= 0 ? ps : 0;
    wj[j] = w[s];
  }
  f32x4_t v[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)   // read once: non-temporal
    v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(o + (size_t)p[j] * H + n));
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (use[j]) {
      a0 = fmaf(wj[j], v[j][0], a0);
      a1 = fmaf(wj[j], v[j][1], a1);
      a2 = fmaf(wj[j], v[j][2], a2);
      a3 = fmaf(wj[j], v[j][3], a3);
    }
  }
  if (OUT_F32) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(y) + (size_t)t * H + n) = f32x4_t{a0, a1, a2, a3};
  } else {
    u32x2_t out = {pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)};
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<bf16_t*>(y) + (size_t)t * H + n) = out;
  }
}

}  // namespace

hipError_t launch_combine(const float* o, const int32_t* pos, const float* w, int64_t T, int H, int k,
                          void* y, hipStream_t stream, bool out_f32) {
  const int64_t items = T * (H / 4);
  dim3 grid((unsigned)((items + kCombineThreads - 1) / kCombineThreads));
  auto kern = out_f32 ? (k <= 4 ? combine_kernel<4, true> : combine_kernel<MOE_MAX_K_DEV, true>)
                      : (k <= 4 ? combine_kernel<4, false> : combine_kernel<MOE_MAX_K_DEV, false>);
  hipLaunchKernelGGL(kern, grid, dim3(kCombineThreads), 0, stream, o, pos, w, T, H, k, y);
  return hipGetLastError();
}

}  // namespace moe
