// MXFP4 expert weights (W4A16): the quantiser and the weight-streaming expert
// kernel for small token counts per expert.
//
// xserv "Phase 19: gpt-oss-20b MoE support", section 5: "MXFP4 W4A16" -- the
// expert weights are 4-bit E2M1 values with one UE8M0 (power-of-two) scale
// per 32 values, activations stay bf16; the page's hand-written dequantising
// GEMV lost on bandwidth efficiency, which is what this kernel is built for.
// Sections 2 and 4 as for the bf16 kernels (per-expert gate_up -> bias -> GLU,
// down -> bias; block-uniform early exits; masked tails).
//
// Layout (K = contraction dimension, N = output columns):
//   codes  uint8 [E][N][K/2]: row n holds the K values of column n, two per
//          byte, k = 2i in bits 0-3 and k = 2i+1 in bits 4-7;
//   scales uint8 [E][N][K/32]: 2^(s - 127) for the 32 values k = 32b..32b+31
//          of column n (s = 255 is NaN).
// E2M1 code: bit 3 sign, bits 2-1 exponent (bias 1), bit 0 mantissa; the
// magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
// streaming variant (non-temporal: each weight byte is read once)
__device__ __forceinline__ u32x4_t buf_ld16_nt(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 2));
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // any offset at or past this reads 0

// ---------------------------------------------------------------------------
// Quantiser: one thread per (expert, column, 32-value block).  The shared
// exponent is floor(log2 max|v|) - 2 (2 = largest E2M1 exponent), clamped to
// [-127, 127]; for a normal maximum floor(log2) is its exponent field minus
// 127, and a zero or subnormal maximum gives the lower clamp.  v / 2^shared
// is exact; it is rounded to the nearest E2M1 magnitude with ties to the even
// code (the thresholds below are the midpoints; a tie goes to the side whose
// code is even) and saturated at 6.
// ---------------------------------------------------------------------------
constexpr int kQThreads = 256;

__device__ __forceinline__ uint32_t e2m1_magnitude_code(float v) {   // v >= 0
  uint32_t c;
  if (v <= 0.25f) c = 0;
  else if (v < 0.75f) c = 1;
  else if (v <= 1.25f) c = 2;
  else if (v < 1.75f) c = 3;
  else if (v <= 2.5f) c = 4;
  else if (v < 3.5f) c = 5;
  else if (v <= 5.0f) c = 6;
  else c = 7;
  return c;
}

__global__ __launch_bounds__(kQThreads) void mxfp4_quantize_kernel(const bf16_t* __restrict__ W, int K, int N,
                                                                    uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales) {
  const int n = blockIdx.x * kQThreads + threadIdx.x;
  const int b = blockIdx.y;
  const int e = blockIdx.z;
  if (n >= N) return;   // no barrier in this kernel
  const bf16_t* src = W + ((size_t)e * K + 32 * (size_t)b) * N + n;
  float v[32];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = bf16_to_f32(src[(size_t)i * N]);
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  const int sbyte = min(max(ex - 2, 0), 254);       // shared exponent + 127
  const int inv = 127 - sbyte;                      // v / 2^(sbyte - 127) = v * 2^inv
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float m = ldexpf(fabsf(v[i]), inv);
    const uint32_t c = e2m1_magnitude_code(m) | ((__float_as_uint(v[i]) >> 31) << 3);
    packed[i / 8] |= c << (4 * (i % 8));
  }
  const size_t row = (size_t)e * N + n;
  *reinterpret_cast<u32x4_t*>(codes + row * (K / 2) + 16 * (size_t)b) =
      u32x4_t{packed[0], packed[1], packed[2], packed[3]};
  scales[row * (K / 32) + b] = (uint8_t)sbyte;
}

// ---------------------------------------------------------------------------
// Weight-streaming expert kernel.  A workgroup owns one expert and a slice of
// 128 output columns; its four waves split K in quads of four 32-value
// blocks (128 K).  Lane (g = lane/16, c = lane%16), call j = 0..7, reads
// block 4q+g of column n0+8c+j: 16 bytes, the whole block.  The four 8-value
// quarters t of that block are the B operands of four
// v_mfma_f32_16x16x32_bf16 calls, K index 32(4q+g) + 8t + i in MFMA K slot
// (g, i); the token operand is loaded in the same order (lane (row, g), 16
// bytes of x at K = 32(4q+g) + 8t).  MFMA column c of call j is weight column
// n0+8c+j, as in the bf16 kernel, so gate and up of one pair (j, j+1) sit in
// the same lane.  The dequantisation is v_cvt_scalef32_pk_bf16_fp4 (two
// codes per instruction, exact for every scale).  The slice's scales are
// staged transposed in LDS ([block][column]), so a lane reads the scales of
// its eight columns with one 8-byte access.
// ---------------------------------------------------------------------------
constexpr int kMxThreads = 256;
constexpr int kMxWaves = 4;
constexpr int kMxCols = 128;
constexpr int64_t kMxOneChunkMeanRows = 10;

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// UE8M0 byte -> float32 scale 2^(s - 127) (s = 0 is the subnormal 2^-127, 255 NaN)
__device__ __forceinline__ float ue8m0_to_f32(uint32_t s) {
  uint32_t u = s << 23;
  u = s == 0 ? 0x00400000u : u;
  u = s == 255 ? 0x7FC00000u : u;
  return __uint_as_float(u);
}

// eight E2M1 codes (one dword, k = 0..7 from the low nibble up) -> eight bf16 * scale
__device__ __forceinline__ u32x4_t dequant8(uint32_t w, float s) {
  const bf16x2_v a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2_v b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2_v c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2_v d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  return u32x4_t{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                 __builtin_bit_cast(uint32_t, d)};
}

template <bool GATE_UP, int MG>
__global__ __launch_bounds__(kMxThreads) void gemv_mxfp4_kernel(
    const bf16_t* __restrict__ A,        // gate_up: x [T][K]; down: h [S][K] in permuted order
    const uint8_t* __restrict__ Wq,      // [E][N][K/2]
    const uint8_t* __restrict__ Ws,      // [E][N][K/32]
    const bf16_t* __restrict__ bias,     // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,    // gate_up only: permuted slot ids
    int K, int N, int kslots, int a_rows, void* __restrict__ out) {
  __shared__ float red[kMxWaves][8][4][kWave];   // 32 KB: one chunk's partial sums per wave
  extern __shared__ __align__(16) uint8_t sc[];  // [K/32][128] scales of the slice

  const int e = blockIdx.y;
  const int M = cnt[e];
  if (M == 0) return;   // block-uniform: no load, no barrier for an expert without rows
  const int row0 = off[e];
  const int nblk = K / 32;
  const int n0 = blockIdx.x * kMxCols;
  const int ncols = min(kMxCols, N - n0);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane >> 4;
  const int c = lane & 15;

  // ---- scales of the slice -> LDS [block][column] ----
  {
    const uint32_t bytes = (uint32_t)ncols * nblk;   // contiguous: rows n0.. of [N][K/32]
    const rsrc_t s_rs = make_rsrc(Ws + ((size_t)e * N + n0) * nblk, bytes);
    // 8-byte pieces: the region starts at a multiple of 8 bytes (N % 8 == 0)
    for (uint32_t p0 = 8u * tid; p0 < bytes; p0 += 8u * kMxThreads) {
      const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(s_rs, (int)p0, 0, 0));
      uint32_t col = p0 / nblk, blk = p0 - col * nblk;   // walked forward byte by byte
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (p0 + q < bytes) sc[blk * kMxCols + col] = (uint8_t)(v[q / 4] >> (8 * (q % 4)));
        ++blk;
        const bool wrap = blk == (uint32_t)nblk;
        blk = wrap ? 0u : blk;
        col += wrap ? 1u : 0u;
      }
    }
  }
  __syncthreads();

  const uint32_t row_bytes = (uint32_t)K / 2;
  const rsrc_t w_rs = make_rsrc(Wq + (size_t)e * N * row_bytes, (uint32_t)N * row_bytes);
  const rsrc_t a_rs = make_rsrc(A, (uint32_t)((size_t)a_rows * K * 2));
  uint32_t w_off[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) w_off[j] = (uint32_t)min(n0 + 8 * c + j, N - 1) * row_bytes;
  const bool col_ok = n0 + 8 * c < N;

  const int nq = (nblk + 3) / 4;
  const int q_begin = (nq * wave) / kMxWaves;
  const int q_end = (nq * (wave + 1)) / kMxWaves;

  for (int r0 = 0; r0 < M; r0 += 16 * MG) {
    const int nch = min(MG, (M - r0 + 15) / 16);   // block-uniform
    uint32_t a_off[MG];
#pragma unroll
    for (int qq = 0; qq < MG; ++qq) {
      const int m = min(r0 + 16 * qq + c, M - 1);   // A row of this lane (clamped)
      const uint32_t r = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
      a_off[qq] = r * (uint32_t)K * 2u;
    }

    f32x4_t acc[MG][8];
#pragma unroll
    for (int qq = 0; qq < MG; ++qq)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[qq][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Loads of quad q into one register set: the lane's block 4q+g of its
    // eight columns and the 4 x MG pieces of token rows.  A block past K (or
    // a quad past this wave's range) is sent outside the descriptors.
    auto load = [&](int q, u32x4_t (&wd)[8], u32x4_t (&ad)[MG][4]) {
      const int b = 4 * q + g;
      const bool in = q < q_end && b < nblk;
#pragma unroll
      for (int j = 0; j < 8; ++j) wd[j] = buf_ld16_nt(w_rs, in ? w_off[j] + 16u * b : kOutOfRange);
#pragma unroll
      for (int qq = 0; qq < MG; ++qq)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          ad[qq][t] = buf_ld16(a_rs, in ? a_off[qq] + (uint32_t)(32 * b + 8 * t) * 2u : kOutOfRange);
    };
    auto step = [&](int q, const u32x4_t (&wd)[8], const u32x4_t (&ad)[MG][4]) {
      const int b = min(4 * q + g, nblk - 1);
      const uint2 s8 = *reinterpret_cast<const uint2*>(sc + b * kMxCols + 8 * c);
      float s[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) s[j] = ue8m0_to_f32(((j < 4 ? s8.x : s8.y) >> (8 * (j & 3))) & 0xFF);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4_t bw = dequant8(wd[j][t], s[j]);
          acc[0][j] = mfma16x16x32(ad[0][t], bw, acc[0][j]);
          if (MG > 1 && nch > 1) {
#pragma unroll
            for (int qq = 1; qq < MG; ++qq) acc[qq][j] = mfma16x16x32(ad[qq][t], bw, acc[qq][j]);
          }
        }
    };

    u32x4_t wcur[8], wnxt[8], acur[MG][4], anxt[MG][4];
    load(q_begin, wcur, acur);
    int q = q_begin;
    for (; q + 2 <= q_end; q += 2) {
      load(q + 1, wnxt, anxt);
      step(q, wcur, acur);
      load(q + 2, wcur, acur);
      step(q + 1, wnxt, anxt);
    }
    if (q < q_end) step(q, wcur, acur);

    // Sum the four K partials (fixed order: wave 0, 1, 2, 3), then the epilogue.
    // Wave w finishes MFMA calls j = 2w and 2w+1 (columns n0+8c+2w, +2w+1).
#pragma unroll
    for (int qq = 0; qq < MG; ++qq) {
      if (qq < nch) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[qq][j][v];
        __syncthreads();
        const int col = n0 + 8 * c + 2 * wave;
        float b0 = 0.f, b1 = 0.f;
        if (col_ok) {
          const uint32_t bw = *reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + col);
          b0 = bf16lo(bw);
          b1 = bf16hi(bw);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = r0 + 16 * qq + 4 * g + v;   // C row held in slot v of this lane
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < kMxWaves; ++w2) {
            s0 += red[w2][2 * wave][v][lane];
            s1 += red[w2][2 * wave + 1][v][lane];
          }
          if (m < M && col_ok) {
            const size_t orow = (size_t)(row0 + m);
            if (GATE_UP) {
              const float hv = clamped_glu(s0 + b0, s1 + b1);
              reinterpret_cast<uint16_t*>(out)[orow * (N / 2) + col / 2] = (uint16_t)f32_to_bf16(hv);
            } else {
              *reinterpret_cast<float2*>(reinterpret_cast<float*>(out) + orow * N + col) =
                  make_float2(s0 + b0, s1 + b1);
            }
          }
        }
        __syncthreads();
      }
    }
  }
}

template <bool GATE_UP>
hipError_t launch_mx(const void* A, const void* Wq, const void* Ws, const void* bias, const int32_t* cnt,
                     const int32_t* off, const int32_t* rows, int64_t T, int K, int N, int E, int k,
                     int64_t a_rows, void* out, hipStream_t stream) {
  // 32-bit buffer offsets: the token operand and one expert's codes below
  // 2 GiB, so an offset at kOutOfRange never wraps back into range
  if (a_rows * K * 2 >= ((int64_t)1 << 31) || (int64_t)N * K / 2 >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  dim3 grid((unsigned)((N + kMxCols - 1) / kMxCols), (unsigned)E);
  const size_t lds = (size_t)(K / 32) * kMxCols;
  const bool one = T * k <= kMxOneChunkMeanRows * E;
  auto kern = one ? gemv_mxfp4_kernel<GATE_UP, 1> : gemv_mxfp4_kernel<GATE_UP, 2>;
  hipLaunchKernelGGL(kern, grid, dim3(kMxThreads), lds, stream, (const bf16_t*)A, (const uint8_t*)Wq,
                     (const uint8_t*)Ws, (const bf16_t*)bias, cnt, off, rows, K, N, GATE_UP ? k : 1, (int)a_rows,
                     out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mxfp4_quantize(const void* W, int E, int K, int N, void* codes, void* scales, hipStream_t stream) {
  dim3 grid((unsigned)((N + kQThreads - 1) / kQThreads), (unsigned)(K / 32), (unsigned)E);
  hipLaunchKernelGGL(mxfp4_quantize_kernel, grid, dim3(kQThreads), 0, stream, (const bf16_t*)W, K, N,
                     (uint8_t*)codes, (uint8_t*)scales);
  return hipGetLastError();
}

hipError_t launch_mxfp4_gate_up(const void* x, const void* Wq, const void* Ws, const void* bgu, const int32_t* cnt,
                                const int32_t* off, const int32_t* rows, int64_t T, int H, int E, int k, int I,
                                void* h, hipStream_t stream) {
  return launch_mx<true>(x, Wq, Ws, bgu, cnt, off, rows, T, H, 2 * I, E, k, T, h, stream);
}

hipError_t launch_mxfp4_down(const void* h, const void* Wq, const void* Ws, const void* bd, const int32_t* cnt,
                             const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                             hipStream_t stream) {
  return launch_mx<false>(h, Wq, Ws, bd, cnt, off, nullptr, T, I, H, E, k, T * k, o, stream);
}

}  // namespace moe
