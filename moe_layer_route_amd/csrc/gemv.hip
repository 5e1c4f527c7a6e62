// Weight-streaming expert GEMMs for small token counts per expert.
//
// xserv "Phase 19: gpt-oss-20b MoE support": section 2 (per-expert gate_up GEMM
// -> bias -> GLU -> down GEMM -> bias; the dense all-expert weight reads are
// the decode cost that a sparse GEMV removes) and section 4 (a workgroup may
// only leave early when the whole workgroup leaves together, before any load
// or barrier; tails of N = 2880, which is not a multiple of 128, are masked).
//
// At decode sizes each expert sees a handful of rows, so the cost is reading
// the expert's weights once from HBM.  A workgroup owns one expert and one
// 128-column slice of its weight; its four waves split K and stream their
// rows of the slice straight from HBM into registers:
//   lane (g = lane/16, c = lane%16) loads rows kb+8g .. kb+8g+7 of the 8
//   columns n0+8c .. n0+8c+7 (eight 16-byte loads),
// then an 8x8 transpose in registers turns them into eight K-packed B
// operands of v_mfma_f32_16x16x32_bf16 (one per column offset j; MFMA column
// c of call j is weight column n0+8c+j).  The A operand is the matching
// 16-byte piece of up to 16 token rows (read from L2).  The four K partial
// sums are added in LDS in a fixed order, then the epilogue adds the bias and
// applies the GLU (gate_up; gate/up columns 2i, 2i+1 are calls j and j+1 of
// the same lane) or writes float32 (down).
//
// Experts with no rows exit before any load.  Rows beyond 32 are handled in
// further passes over the weights (only under heavy routing skew).
//
// All operand loads are unconditional buffer loads (a masked load becomes a
// branch, and the compiler then drains every outstanding load at the merge,
// which would serialise the prefetch).  Rows past M and columns past N read a
// valid row or column instead -- they only feed outputs that are never
// stored -- and the K tail and the prefetch past a wave's K range are sent
// outside the buffer descriptors, which read as 0 without touching memory.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kGvThreads = 256;
constexpr int kGvWaves = 4;
constexpr int kGvCols = 128;   // weight columns per workgroup
constexpr int kGvKB = 32;      // K rows per MFMA step

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// streaming variant (non-temporal: each weight byte is read once)
__device__ __forceinline__ u32x4_t buf_ld16_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // any offset at or past this reads 0
// Mean rows per expert up to which one 16-row chunk per pass is used (an
// expert with more rows takes extra passes over its weights).
constexpr int64_t kGvOneChunkMeanRows = 10;

// MG = 16-row chunks per pass over the weights (1 or 2, picked from the mean
// rows per expert: more chunks mean fewer passes but more accumulators).
template <bool GATE_UP, int MG>
__global__ __launch_bounds__(kGvThreads) void gemv_expert_kernel(
    const bf16_t* __restrict__ A,      // gate_up: x [T][K]; down: h [S][K] in permuted order
    const bf16_t* __restrict__ W,      // [E][K][N]
    const bf16_t* __restrict__ bias,   // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,  // gate_up only: permuted slot ids
    int K, int N, int kslots, int a_rows, void* __restrict__ out) {
  __shared__ float red[kGvWaves][8][4][kWave];   // 32 KB: one chunk's partial sums per wave

  const int e = blockIdx.y;
  const int M = cnt[e];
  if (M == 0) return;   // block-uniform: no load, no barrier for an expert without rows
  const int row0 = off[e];

  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform, stated so: it feeds scalar (soffset) operands
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int c = lane & 15;
  const int ncol = blockIdx.x * kGvCols + 8 * c;
  const bool col_ok = ncol < N;
  const rsrc_t w_rs = make_rsrc(W + (size_t)e * K * N, (uint32_t)((size_t)K * N * 2));
  const rsrc_t a_rs = make_rsrc(A, (uint32_t)((size_t)a_rows * K * 2));
  const uint32_t w_col = (uint32_t)min(ncol, N - 8);

  const int nkb = (K + kGvKB - 1) / kGvKB;
  const int kb_begin = (nkb * wave) / kGvWaves;
  const int kb_end = (nkb * (wave + 1)) / kGvWaves;

  for (int r0 = 0; r0 < M; r0 += 16 * MG) {
    const int nch = min(MG, (M - r0 + 15) / 16);   // block-uniform
    uint32_t a_off[MG];
#pragma unroll
    for (int q = 0; q < MG; ++q) {
      const int m = min(r0 + 16 * q + c, M - 1);   // A row of this lane (clamped)
      const uint32_t r = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
      a_off[q] = (r * (uint32_t)K + 8u * g) * 2u;
    }

    f32x4_t acc[MG][8];
#pragma unroll
    for (int q = 0; q < MG; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[q][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wcur[8], wnxt[8], acur[MG], anxt[MG];
    // Loads of K block kb.  The K-block offset is wave-uniform and goes into
    // the scalar offset; blocks outside [kb_begin, kb_end) (a uniform test)
    // and rows past K fall outside the descriptor and read 0.
    const uint32_t w_voff = ((uint32_t)(8 * g) * N + w_col) * 2u;
    auto load = [&](int kb, u32x4_t (&wd)[8], u32x4_t (&ad)[MG]) {
      const bool in = kb < kb_end;
      const uint32_t w_soff = in ? (uint32_t)(kb * kGvKB) * N * 2u : kOutOfRange;
#pragma unroll
      for (int r = 0; r < 8; ++r) wd[r] = buf_ld16_nt(w_rs, w_voff + (uint32_t)r * N * 2u, w_soff);
      const bool a_in = kb * kGvKB + 8 * g < K;
      const uint32_t a_soff = in ? 64u * kb : kOutOfRange;
#pragma unroll
      for (int q = 0; q < MG; ++q) ad[q] = buf_ld16(a_rs, a_in ? a_off[q] : kOutOfRange, a_soff);
    };

    // one K block: prefetch the next into the other register set, then
    // transpose and multiply the current one (two sets, ping-pong, so no
    // register copy waits on the loads in flight)
    auto step = [&](int kb, u32x4_t (&wc)[8], u32x4_t (&ac)[MG], u32x4_t (&wn)[8], u32x4_t (&an)[MG]) {
      load(kb + 1, wn, an);
      u32x4_t bt[8];
      transpose8x8_b16(wc, bt);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[0][j] = mfma16x16x32(ac[0], bt[j], acc[0][j]);
      if (MG > 1 && nch > 1) {
#pragma unroll
        for (int q = 1; q < MG; ++q)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[q][j] = mfma16x16x32(ac[q], bt[j], acc[q][j]);
      }
    };
    load(kb_begin, wcur, acur);
    int kb = kb_begin;
    for (; kb + 2 <= kb_end; kb += 2) {
      step(kb, wcur, acur, wnxt, anxt);
      step(kb + 1, wnxt, anxt, wcur, acur);
    }
    if (kb < kb_end) step(kb, wcur, acur, wnxt, anxt);

    // Sum the four K partials (fixed order: wave 0, 1, 2, 3), then the epilogue.
    // Wave w finishes MFMA calls j = 2w and 2w+1 (columns ncol+2w, ncol+2w+1).
#pragma unroll
    for (int q = 0; q < MG; ++q) {
      if (q < nch) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[q][j][v];
        __syncthreads();
        const int col = ncol + 2 * wave;
        float b0 = 0.f, b1 = 0.f;
        if (col_ok) {
          const uint32_t bw = *reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + col);
          b0 = bf16lo(bw);
          b1 = bf16hi(bw);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = r0 + 16 * q + 4 * g + v;   // C row held in slot v of this lane
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < kGvWaves; ++w2) {
            s0 += red[w2][2 * wave][v][lane];
            s1 += red[w2][2 * wave + 1][v][lane];
          }
          if (m < M && col_ok) {
            const size_t orow = (size_t)(row0 + m);
            if (GATE_UP) {
              const float hv = clamped_glu(s0 + b0, s1 + b1);
              reinterpret_cast<uint16_t*>(out)[orow * (N / 2) + col / 2] = (uint16_t)f32_to_bf16(hv);
            } else {
              float2 ov = make_float2(s0 + b0, s1 + b1);
              *reinterpret_cast<float2*>(reinterpret_cast<float*>(out) + orow * N + col) = ov;
            }
          }
        }
        __syncthreads();
      }
    }
  }
}

}  // namespace

hipError_t launch_gemv_gate_up(const void* x, const void* Wgu, const void* bgu, const int32_t* cnt,
                               const int32_t* off, const int32_t* rows, int64_t T, int H, int E, int k, int I,
                               void* h, hipStream_t stream) {
  const int N = 2 * I;
  // buffer offsets: x and one expert's weight (plus the K-tail overrun) below
  // 2 GiB, so an offset pushed past kOutOfRange never wraps back into range
  if (T * H * 2 >= ((int64_t)1 << 31) || (int64_t)(H + 64) * N * 2 >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  dim3 grid((unsigned)((N + kGvCols - 1) / kGvCols), (unsigned)E);
  auto kern = T * k <= kGvOneChunkMeanRows * E ? gemv_expert_kernel<true, 1> : gemv_expert_kernel<true, 2>;
  hipLaunchKernelGGL(kern, grid, dim3(kGvThreads), 0, stream, (const bf16_t*)x,
                     (const bf16_t*)Wgu, (const bf16_t*)bgu, cnt, off, rows, H, N, k, (int)T, h);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const void* h, const void* Wd, const void* bd, const int32_t* cnt,
                            const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                            hipStream_t stream) {
  const int64_t S = T * k;
  if (S * I * 2 >= ((int64_t)1 << 31) || (int64_t)(I + 64) * H * 2 >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  dim3 grid((unsigned)((H + kGvCols - 1) / kGvCols), (unsigned)E);
  auto kern = T * k <= kGvOneChunkMeanRows * E ? gemv_expert_kernel<false, 1> : gemv_expert_kernel<false, 2>;
  hipLaunchKernelGGL(kern, grid, dim3(kGvThreads), 0, stream, (const bf16_t*)h,
                     (const bf16_t*)Wd, (const bf16_t*)bd, cnt, off, (const int32_t*)nullptr, I, H, 1, (int)S,
                     (void*)o);
  return hipGetLastError();
}

}  // namespace moe
