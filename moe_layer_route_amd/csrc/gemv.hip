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
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kGvThreads = 256;
constexpr int kGvWaves = 4;
constexpr int kGvCols = 128;   // weight columns per workgroup
constexpr int kGvKB = 32;      // K rows per MFMA step
constexpr int kGvMG = 2;       // 16-row chunks per pass

template <bool GATE_UP>
__global__ __launch_bounds__(kGvThreads) void gemv_expert_kernel(
    const bf16_t* __restrict__ A,      // gate_up: x [T][K]; down: h [S][K] in permuted order
    const bf16_t* __restrict__ W,      // [E][K][N]
    const bf16_t* __restrict__ bias,   // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,  // gate_up only: permuted slot ids
    int K, int N, int kslots, void* __restrict__ out) {
  __shared__ float red[kGvWaves][8][4][kWave];   // 32 KB: one chunk's partial sums per wave

  const int e = blockIdx.y;
  const int M = cnt[e];
  if (M == 0) return;   // block-uniform: no load, no barrier for an expert without rows
  const int row0 = off[e];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int ncol = blockIdx.x * kGvCols + 8 * c;
  const bool col_ok = ncol < N;
  const bf16_t* __restrict__ We = W + (size_t)e * K * N + ncol;

  const int nkb = (K + kGvKB - 1) / kGvKB;
  const int kb_begin = (nkb * wave) / kGvWaves;
  const int kb_end = (nkb * (wave + 1)) / kGvWaves;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  for (int r0 = 0; r0 < M; r0 += 16 * kGvMG) {
    const int nch = min(kGvMG, (M - r0 + 15) / 16);   // block-uniform
    const bf16_t* arow[kGvMG];
    bool aok[kGvMG];
#pragma unroll
    for (int q = 0; q < kGvMG; ++q) {
      const int m = r0 + 16 * q + c;   // A row of this lane
      aok[q] = m < M;
      size_t r = 0;
      if (aok[q]) r = GATE_UP ? (size_t)(rows[row0 + m] / kslots) : (size_t)(row0 + m);
      arow[q] = A + r * K + 8 * g;
    }

    f32x4_t acc[kGvMG][8];
#pragma unroll
    for (int q = 0; q < kGvMG; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[q][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wcur[8], wnxt[8], acur[kGvMG], anxt[kGvMG];
    auto load_w = [&](int kb, u32x4_t (&dst)[8]) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int kr = kb * kGvKB + 8 * g + r;
        dst[r] = (col_ok && kr < K) ? ldg16_stream(We + (size_t)kr * N) : zero;
      }
    };
    auto load_a = [&](int kb, u32x4_t (&dst)[kGvMG]) {
      const int k0 = kb * kGvKB + 8 * g;
#pragma unroll
      for (int q = 0; q < kGvMG; ++q) dst[q] = (aok[q] && k0 < K) ? ld16(arow[q] + kb * kGvKB) : zero;
    };

    if (kb_begin < kb_end) {
      load_w(kb_begin, wcur);
      load_a(kb_begin, acur);
    }
    for (int kb = kb_begin; kb < kb_end; ++kb) {
      if (kb + 1 < kb_end) {
        load_w(kb + 1, wnxt);
        load_a(kb + 1, anxt);
      }
      u32x4_t bt[8];
      transpose8x8_b16(wcur, bt);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[0][j] = mfma16x16x32(acur[0], bt[j], acc[0][j]);
      if (nch > 1) {
#pragma unroll
        for (int q = 1; q < kGvMG; ++q)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[q][j] = mfma16x16x32(acur[q], bt[j], acc[q][j]);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) wcur[r] = wnxt[r];
#pragma unroll
      for (int q = 0; q < kGvMG; ++q) acur[q] = anxt[q];
    }

    // Sum the four K partials (fixed order: wave 0, 1, 2, 3), then the epilogue.
    // Wave w finishes MFMA calls j = 2w and 2w+1 (columns ncol+2w, ncol+2w+1).
#pragma unroll
    for (int q = 0; q < kGvMG; ++q) {
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
                               const int32_t* off, const int32_t* rows, int H, int E, int k, int I,
                               void* h, int max_rows_hint, hipStream_t stream) {
  (void)max_rows_hint;
  const int N = 2 * I;
  dim3 grid((unsigned)((N + kGvCols - 1) / kGvCols), (unsigned)E);
  hipLaunchKernelGGL(gemv_expert_kernel<true>, grid, dim3(kGvThreads), 0, stream, (const bf16_t*)x,
                     (const bf16_t*)Wgu, (const bf16_t*)bgu, cnt, off, rows, H, N, k, h);
  return hipGetLastError();
}

hipError_t launch_gemv_down(const void* h, const void* Wd, const void* bd, const int32_t* cnt,
                            const int32_t* off, int H, int E, int I, float* o, int max_rows_hint,
                            hipStream_t stream) {
  (void)max_rows_hint;
  dim3 grid((unsigned)((H + kGvCols - 1) / kGvCols), (unsigned)E);
  hipLaunchKernelGGL(gemv_expert_kernel<false>, grid, dim3(kGvThreads), 0, stream, (const bf16_t*)h,
                     (const bf16_t*)Wd, (const bf16_t*)bd, cnt, off, (const int32_t*)nullptr, I, H, 1,
                     (void*)o);
  return hipGetLastError();
}

}  // namespace moe
