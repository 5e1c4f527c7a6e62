// Router of the gpt-oss MoE block: logits, top-k, softmax weights.
//
// xserv "Phase 19: gpt-oss-20b MoE support", section 1 ("MoE" row: the router
// is a plain Linear with bias) and section 2 (router -> top-k softmax, with the
// expert ids staying on the device).
//
// One workgroup per token.  The token's row of x is staged in LDS; each wave
// owns every fourth expert and accumulates its dot product in float64 (the
// bf16 x bf16 products are exact in float64, so the only rounding is the
// float64 accumulation, ~1e-16 relative).  The logit plus bias is rounded to
// float32 and the top-k decision is taken on those float32 values with the
// ordering key (value desc, index asc).  The softmax over the k selected
// experts uses the float64 logits.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;

// Monotone map of float32 to uint32 (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = __shfl_xor(v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, const bf16_t* __restrict__ br,
    int H, int E, int k, int32_t* __restrict__ ids, float* __restrict__ wout) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* logit = reinterpret_cast<double*>(smem);                                  // [E]
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem + sizeof(double) * MOE_MAX_E_DEV);     // [H]

  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nchunk = H / 8;   // 16-byte chunks of a row

  const bf16_t* xrow = x + (size_t)t * H;
  for (int c = threadIdx.x; c < nchunk; c += kRouteThreads)
    *reinterpret_cast<u32x4_t*>(xs + 8 * c) = ld16(xrow + 8 * c);
  __syncthreads();

  // Each wave takes experts wave, wave + 4, ... in groups of 4.
  for (int e0 = wave * 4; e0 < E; e0 += kRouteWaves * 4) {
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int c = lane; c < nchunk; c += kWave) {
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + 8 * c);
      double xd[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xd[2 * q] = (double)bf16lo(xv[q]);
        xd[2 * q + 1] = (double)bf16hi(xv[q]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + i;
        if (e < E) {
          const u32x4_t wv = ld16(Wr + (size_t)e * H + 8 * c);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[i] = fma(xd[2 * q], (double)bf16lo(wv[q]), acc[i]);
            acc[i] = fma(xd[2 * q + 1], (double)bf16hi(wv[q]), acc[i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double s = wave_sum(acc[i]);
      const int e = e0 + i;
      if (lane == 0 && e < E) logit[e] = s + (double)bf16_to_f32(br[e]);
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // Top-k over float32-rounded logits.  Each lane owns experts lane + 64*i.
  uint64_t key[MOE_MAX_E_DEV / kWave];
#pragma unroll
  for (int i = 0; i < MOE_MAX_E_DEV / kWave; ++i) {
    const int e = lane + kWave * i;
    key[i] = 0;   // below every real key (real keys have a non-zero low word)
    if (e < E) {
      const float v = (float)logit[e];
      key[i] = ((uint64_t)order_key(v) << 32) | (uint64_t)(0xFFFFu - (uint32_t)e);
    }
  }
  int sel[MOE_MAX_K_DEV];
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < MOE_MAX_E_DEV / kWave; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFu - (uint32_t)(best & 0xFFFFu));
    sel[j] = e;
#pragma unroll
    for (int i = 0; i < MOE_MAX_E_DEV / kWave; ++i)
      if (lane + kWave * i == e) key[i] = 0;
  }
  if (lane == 0) {
    const double l0 = logit[sel[0]];
    double z[MOE_MAX_K_DEV];
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
      z[j] = exp(logit[sel[j]] - l0);
      sum += z[j];
    }
    for (int j = 0; j < k; ++j) {
      ids[(size_t)t * k + j] = sel[j];
      wout[(size_t)t * k + j] = (float)(z[j] / sum);
    }
  }
}

}  // namespace

hipError_t launch_route(const void* x, const void* Wr, const void* br, int64_t T, int H, int E, int k,
                        int32_t* ids, float* w, hipStream_t stream) {
  const size_t lds = sizeof(double) * MOE_MAX_E_DEV + sizeof(bf16_t) * (size_t)H;
  hipLaunchKernelGGL(route_kernel, dim3((unsigned)T), dim3(kRouteThreads), lds, stream,
                     (const bf16_t*)x, (const bf16_t*)Wr, (const bf16_t*)br, H, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
