// Expert-contiguous permutation of the T*k (token, slot) pairs.
//
// xserv "Phase 19: gpt-oss-20b MoE support", section 2: the dense pipeline
// copies every token to every local expert; the sparse formulation instead
// groups the (token, slot) pairs by expert so that each expert reads only the
// rows routed to it.  The expert ids never leave the device, so this counting
// sort runs on the GPU and everything downstream reads cnt/off from device
// memory.
//
// One workgroup of 16 waves.  Wave w owns a contiguous range of slots.
// Pass 1 counts the range per expert (integer LDS atomics: the counts do not
// depend on the order).  Wave 0 scans the totals; each expert's per-wave base
// is its offset plus the counts of the earlier waves.  Pass 2 walks each range
// again in order, 64 slots at a time: the lanes that share an expert are found
// with eight ballots over the bits of the id, a lane's rank among them is the
// popcount of the lower lanes, and the lowest lane of the group advances the
// wave's base for that expert.  The result is the stable order (by slot
// index) and is identical on every run.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int S, int E, int32_t* __restrict__ cnt,
    int32_t* __restrict__ off, int32_t* __restrict__ rows, int32_t* __restrict__ pos) {
  __shared__ int hist[kPermWaves][MOE_MAX_E_DEV];
  __shared__ int offs[MOE_MAX_E_DEV];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  for (int i = tid; i < kPermWaves * MOE_MAX_E_DEV; i += kPermThreads) (&hist[0][0])[i] = 0;
  __syncthreads();

  const int per = (S + kPermWaves - 1) / kPermWaves;
  const int s_begin = min(S, wave * per);
  const int s_end = min(S, s_begin + per);

  for (int s = s_begin + lane; s < s_end; s += kWave) atomicAdd(&hist[wave][ids[s]], 1);
  __syncthreads();

  if (wave == 0) {
    int c[4];
    int tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      int v = 0;
      if (e < E)
        for (int w = 0; w < kPermWaves; ++w) v += hist[w][e];
      c[i] = v;
      tot += v;
    }
    const int incl = wave_inclusive_scan(tot, lane);
    int run = incl - tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < E) {
        offs[e] = run;
        cnt[e] = c[i];
        off[e] = run;
      }
      run += c[i];
    }
    if (lane == kWave - 1) off[E] = incl;
  }
  __syncthreads();
  if (tid < E) {
    int run = offs[tid];
    for (int w = 0; w < kPermWaves; ++w) {
      const int h = hist[w][tid];
      hist[w][tid] = run;
      run += h;
    }
  }
  __syncthreads();

  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  for (int sb = s_begin; sb < s_end; sb += kWave) {
    const int s = sb + lane;
    const bool valid = s < s_end;
    const int e = valid ? ids[s] : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int leader = __ffsll((unsigned long long)peers) - 1;
    int base = 0;
    if (valid && lane == leader) {
      base = hist[wave][e];
      hist[wave][e] = base + __popcll(peers);
    }
    base = __shfl(base, leader < 0 ? 0 : leader, kWave);
    if (valid) {
      const int p = base + __popcll(peers & lt_mask);
      rows[p] = s;
      pos[s] = p;
    }
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int64_t T, int E, int k, int32_t* cnt, int32_t* off,
                          int32_t* rows, int32_t* pos, hipStream_t stream) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, ids, (int)(T * k), E, cnt,
                     off, rows, pos);
  return hipGetLastError();
}

}  // namespace moe
