// Expert-contiguous permutation of the T*k (token, slot) pairs.
//
// xserv "Phase 19: gpt-oss-20b MoE support", section 2: the dense pipeline
// copies every token to every local expert; the sparse formulation instead
// groups the (token, slot) pairs by expert so that each expert reads only the
// rows routed to it.  The expert ids never leave the device, so this counting
// sort runs on the GPU and everything downstream reads cnt/off from device
// memory.
//
// The slots are cut into chunks of kPermChunk, one workgroup each.  With a
// single chunk one launch does everything.  With several:
//   1. permute_hist_kernel: each workgroup counts its chunk per expert and
//      writes the counts to pos[], which is free until the last step;
//   2. permute_kernel: each workgroup sums those counts into the totals
//      (cnt, and off by a scan; workgroup 0 writes both) and into the number
//      of earlier slots per expert in earlier chunks, which is where its own
//      slots of each expert start, then scatters its chunk;
//   3. permute_inverse_kernel: pos[rows[p]] = p.
// Inside a workgroup of 16 waves, wave w owns a contiguous range of the
// chunk.  Pass 1 counts the range per expert (integer LDS atomics: the counts
// do not depend on the order).  Each expert's per-wave base is the chunk's
// base plus the counts of the earlier waves.  Pass 2 walks each range again in
// order, 64 slots at a time: the lanes that share an expert are found with
// eight ballots over the bits of the id, a lane's rank among them is the
// popcount of the lower lanes, and the lowest lane of the group advances the
// wave's base for that expert.  The result is the stable order (by slot
// index) and is identical on every run, whatever the number of chunks.
// Experts are counted from e_begin: slot s goes to local expert
// ids[s] - e_begin, and a slot whose local expert is outside [0, E) is
// skipped and gets pos = -1 (an expert-parallel rank keeps only the experts
// it holds; with e_begin = 0 and every id in [0, E) nothing is skipped).
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / kWave;
constexpr int kPermChunk = 4096;     // slots per workgroup when there are several
constexpr int kPermHistThreads = 256;

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

__global__ __launch_bounds__(kPermHistThreads) void permute_hist_kernel(const int32_t* __restrict__ ids, int S,
                                                                         int e_begin, int E,
                                                                         int32_t* __restrict__ hist) {
  __shared__ int h[MOE_MAX_E_DEV];
  for (int e = threadIdx.x; e < MOE_MAX_E_DEV; e += kPermHistThreads) h[e] = 0;
  __syncthreads();
  const int s_begin = blockIdx.x * kPermChunk;
  const int s_end = min(S, s_begin + kPermChunk);
  // all of a thread's ids are loaded before any is counted
  constexpr int kPer = kPermChunk / kPermHistThreads;
  int e[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int s = s_begin + threadIdx.x + kPermHistThreads * i;
    e[i] = s < s_end ? ids[s] - e_begin : -1;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if ((unsigned)e[i] < (unsigned)E) atomicAdd(&h[e[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermHistThreads) hist[blockIdx.x * E + e] = h[e];
}

// hist: the per-chunk counts (nchunks > 1), or null for a single chunk, which
// then also writes pos.
__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ ids, int S, int e_begin, int E, const int32_t* __restrict__ hist, int nchunks,
    int32_t* __restrict__ cnt, int32_t* __restrict__ off, int32_t* __restrict__ rows, int32_t* __restrict__ pos) {
  __shared__ int whist[kPermWaves][MOE_MAX_E_DEV];
  __shared__ int base[MOE_MAX_E_DEV];
  __shared__ int tot_s[MOE_MAX_E_DEV];   // per expert: all chunks
  __shared__ int pre_s[MOE_MAX_E_DEV];   //             earlier chunks

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  for (int i = tid; i < kPermWaves * MOE_MAX_E_DEV; i += kPermThreads) (&whist[0][0])[i] = 0;
  if (tid < MOE_MAX_E_DEV) tot_s[tid] = pre_s[tid] = 0;
  __syncthreads();
  // the per-chunk counts, summed by all threads (integer atomics: the sums do
  // not depend on the order)
  if (hist != nullptr)
    for (int i = tid; i < nchunks * E; i += kPermThreads) {
      const int v = hist[i];
      atomicAdd(&tot_s[i % E], v);
      if (i / E < (int)blockIdx.x) atomicAdd(&pre_s[i % E], v);
    }

  const int c_begin = blockIdx.x * kPermChunk;
  const int c_len = min(S - c_begin, nchunks > 1 ? kPermChunk : S);
  const int per = (c_len + kPermWaves - 1) / kPermWaves;
  const int s_begin = c_begin + min(c_len, wave * per);
  const int s_end = c_begin + min(c_len, wave * per + per);

  for (int s = s_begin + lane; s < s_end; s += kWave) {
    const int e = ids[s] - e_begin;
    if ((unsigned)e < (unsigned)E) atomicAdd(&whist[wave][e], 1);
  }
  __syncthreads();

  // totals per expert, their exclusive scan (off) and this chunk's base
  if (wave == 0) {
    int tot[4], pre[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      int t = 0, p = 0;
      if (e < E) {
        if (hist != nullptr) {
          t = tot_s[e];
          p = pre_s[e];
        } else {
          for (int w = 0; w < kPermWaves; ++w) t += whist[w][e];
        }
      }
      tot[i] = t;
      pre[i] = p;
      sum += t;
    }
    const int incl = wave_inclusive_scan(sum, lane);
    int run = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      if (e < E) {
        base[e] = run + pre[i];
        if (blockIdx.x == 0) {
          cnt[e] = tot[i];
          off[e] = run;
        }
      }
      run += tot[i];
    }
    if (blockIdx.x == 0 && lane == kWave - 1) off[E] = incl;
  }
  __syncthreads();
  if (tid < E) {
    int run = base[tid];
    for (int w = 0; w < kPermWaves; ++w) {
      const int h = whist[w][tid];
      whist[w][tid] = run;
      run += h;
    }
  }
  __syncthreads();

  const bool write_pos = hist == nullptr;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  for (int sb = s_begin; sb < s_end; sb += kWave) {
    const int s = sb + lane;
    const int id = s < s_end ? ids[s] - e_begin : -1;
    const bool valid = (unsigned)id < (unsigned)E;   // slots outside [0, E) are skipped
    const int e = valid ? id : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bal = __ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int leader = __ffsll((unsigned long long)peers) - 1;
    int wbase = 0;
    if (valid && lane == leader) {
      wbase = whist[wave][e];
      whist[wave][e] = wbase + __popcll(peers);
    }
    wbase = __shfl(wbase, leader < 0 ? 0 : leader, kWave);
    if (valid) {
      const int p = wbase + __popcll(peers & lt_mask);
      rows[p] = s;
      if (write_pos) pos[s] = p;
    } else if (write_pos && s < s_end) {
      pos[s] = -1;
    }
  }
}

// rows[0 .. off[E]) are the written entries; every other slot is a skipped
// one.  The two kinds of writes go to different slots.
__global__ __launch_bounds__(256) void permute_inverse_kernel(const int32_t* __restrict__ ids, int S, int e_begin,
                                                              const int32_t* __restrict__ rows,
                                                              const int32_t* __restrict__ off, int E,
                                                              int32_t* __restrict__ pos) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < S && (unsigned)(ids[i] - e_begin) >= (unsigned)E) pos[i] = -1;
  if (i < off[E]) pos[rows[i]] = i;
}

// Padding rows of a statically sized batch: slots of tokens t >= *n_valid
// (read on the device, clamped to [0, T]) get id -1 and weight 0, so the
// permutation skips them (pos = -1) and no expert ever sees them.
__global__ void mask_padding_kernel(int32_t* __restrict__ ids, float* __restrict__ w, int64_t T, int k,
                                    const int32_t* __restrict__ n_valid) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * k) return;
  const int64_t nv = min(max((int64_t)*n_valid, (int64_t)0), T);
  if (i / k >= nv) {
    ids[i] = -1;
    w[i] = 0.0f;
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* ids, int64_t T, int E, int k, int32_t* cnt, int32_t* off,
                          int32_t* rows, int32_t* pos, hipStream_t stream, int e_begin) {
  const int S = (int)(T * k);
  // one chunk up to kMultiMin slots; above, the per-chunk counts (nchunks x E
  // <= S/16 + 256 <= S entries) fit in pos
  constexpr int kMultiMin = 4 * kPermChunk;
  if (S < kMultiMin) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, ids, S, e_begin, E,
                       (const int32_t*)nullptr, 1, cnt, off, rows, pos);
    return hipGetLastError();
  }
  const int nchunks = (S + kPermChunk - 1) / kPermChunk;
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nchunks), dim3(kPermHistThreads), 0, stream, ids, S, e_begin, E,
                     pos);
  hipLaunchKernelGGL(permute_kernel, dim3(nchunks), dim3(kPermThreads), 0, stream, ids, S, e_begin, E,
                     (const int32_t*)pos, nchunks, cnt, off, rows, (int32_t*)nullptr);
  hipLaunchKernelGGL(permute_inverse_kernel, dim3((S + 255) / 256), dim3(256), 0, stream, ids, S, e_begin,
                     (const int32_t*)rows, (const int32_t*)off, E, pos);
  return hipGetLastError();
}

hipError_t launch_mask_padding(int32_t* ids, float* w, int64_t T, int k, const int32_t* n_valid,
                               hipStream_t stream) {
  const int64_t n = T * k;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mask_padding_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, ids, w, T, k,
                     n_valid);
  return hipGetLastError();
}

}  // namespace moe
