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
//   scales uint8 [E][K/32][N]: scales[e][b][n] = s gives 2^(s - 127) for the
//          32 values k = 32b..32b+31 of column n (s = 255 is NaN).
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
  scales[((size_t)e * (K / 32) + b) * N + n] = (uint8_t)sbyte;
}

// ---------------------------------------------------------------------------
// Weight-streaming expert kernel.  A workgroup owns one expert and a slice of
// 64 output columns; its four waves split K and stream their part straight
// from HBM; the four partial sums are added in LDS in a fixed order.  K is
// walked in double steps of eight 32-value blocks (256 K, one 128-byte line
// of each column).
//   Operands: lane (g = lane/16, c = lane%16), call j = 0..3, uses block
//   8d + 4u + g (u = 0, 1) of column n0+4c+j in double step d: 16 bytes, the
//   whole block, whose four 8-value quarters t are the B operands of four
//   v_mfma_f32_16x16x32_bf16 calls, K index 32(8d+4u+g) + 8t + i in MFMA K
//   slot (g, i); the token operand is loaded in the same order (lane (row,
//   g), 16 bytes of x at K = 32(8d+4u+g) + 8t).  MFMA column c of call j is
//   weight column n0+4c+j, so gate and up of one pair (calls j, j+1) sit in
//   the same lane.  The scales of the lane's four columns for a block are one
//   4-byte load (scales are block-major); v_cvt_scalef32_pk_bf16_fp4
//   dequantises two codes per instruction, exactly for every scale.
//   Weight loads are line-coalesced instead of operand-shaped (eight lanes
//   per 128-byte line: load i, lane L reads block 8d + L%8 of column 8i +
//   L/8), two double steps ahead in a ring of three register sets (with the
//   scales of the same double step; the token rows, from L2, run one 128-K
//   half step ahead in a pair of register sets); each double step
//   writes its codes into the wave's own 8 KB LDS slab and reads back the
//   operand layout.  Slab address of (column, block piece p): column * 128 +
//   16 (p ^ ((column / 4) % 8)): conflict-free writes, at most two-way reads.
// ---------------------------------------------------------------------------
constexpr int kMxWaves = 4;
constexpr int kMxNJ = 4;                 // columns per lane (calls j)
constexpr int kMxCols = 16 * kMxNJ;      // 64 columns per workgroup
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

// one double step's weight loads: 8 coalesced code pieces and the scales of
// the lane's two blocks (u = 0, 1)
struct MxSlot {
  u32x4_t w[8];
  uint32_t s[2];
};
// the token pieces of one half step (block 4q + g)
template <int MG>
struct MxA {
  u32x4_t a[MG][4];
};

template <bool GATE_UP, int MG>
__global__ __launch_bounds__(kMxWaves * kWave) __attribute__((amdgpu_waves_per_eu(MG == 1 ? 2 : 1)))
void gemv_mxfp4_kernel(
    const bf16_t* __restrict__ A,        // gate_up: x [T][K]; down: h [S][K] in permuted order
    const uint8_t* __restrict__ Wq,      // [E][N][K/2]
    const uint8_t* __restrict__ Ws,      // [E][K/32][N]
    const bf16_t* __restrict__ bias,     // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,    // gate_up only: permuted slot ids
    int K, int N, int kslots, int a_rows, void* __restrict__ out) {
  __shared__ float red[kMxWaves][kMxNJ][4][kWave];              // 16 KB: one chunk's partial sums per wave
  __shared__ __align__(16) u32x4_t slab[kMxWaves][kMxCols * 8];  // 32 KB: each wave's staged double step

  const int e = blockIdx.y;
  const int M = cnt[e];
  if (M == 0) return;   // block-uniform: no load, no barrier for an expert without rows
  const int row0 = off[e];
  const int nblk = K / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int c = lane & 15;
  // N % 8 == 0 and ncol % 4 == 0: a lane's four columns are all in range or all out
  const int ncol = blockIdx.x * kMxCols + kMxNJ * c;
  const bool col_ok = ncol < N;

  const uint32_t row_bytes = (uint32_t)K / 2;
  const rsrc_t w_rs = make_rsrc(Wq + (size_t)e * N * row_bytes, (uint32_t)N * row_bytes);
  const rsrc_t s_rs = make_rsrc(Ws + (size_t)e * nblk * N, (uint32_t)(nblk * N));
  const rsrc_t a_rs = make_rsrc(A, (uint32_t)((size_t)a_rows * K * 2));
  const uint32_t s_col = (uint32_t)min(ncol, N - kMxNJ);
  // coalesced code loads: load i covers slab columns 8i .. 8i+7
  const int wl_col = lane >> 3, wl_p = lane & 7;
  uint32_t w_off[8];
  int w_dst[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int col = 8 * i + wl_col;
    w_off[i] = (uint32_t)min(blockIdx.x * kMxCols + col, N - 1) * row_bytes + 16u * wl_p;
    w_dst[i] = col * 8 + (wl_p ^ ((col >> 2) & 7));
  }
  // operand reads: call j, block u of lane (c, g) = column 4c + j, piece 4u + g
  int r_src[kMxNJ][2];
#pragma unroll
  for (int j = 0; j < kMxNJ; ++j)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int col = 4 * c + j;
      r_src[j][u] = col * 8 + ((4 * u + g) ^ ((col >> 2) & 7));
    }
  u32x4_t* const my_slab = slab[wave];
  const int nds = (nblk + 7) / 8;
  const int ds_begin = (nds * wave) / kMxWaves;
  const int ds_end = (nds * (wave + 1)) / kMxWaves;

  for (int r0 = 0; r0 < M; r0 += 16 * MG) {
    const int nch = min(MG, (M - r0 + 15) / 16);   // block-uniform
    uint32_t a_off[MG];
#pragma unroll
    for (int qq = 0; qq < MG; ++qq) {
      const int m = min(r0 + 16 * qq + c, M - 1);   // A row of this lane (clamped)
      const uint32_t r = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
      a_off[qq] = r * (uint32_t)K * 2u;
    }
    f32x4_t acc[MG][kMxNJ];
#pragma unroll
    for (int qq = 0; qq < MG; ++qq)
#pragma unroll
      for (int j = 0; j < kMxNJ; ++j) acc[qq][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // loads of double step d (weights) and half step q (tokens); steps
    // outside this wave's range and blocks past K read 0 (sent outside the
    // descriptors, no memory touched)
    auto load = [&](int d, MxSlot& sl) {
      const bool w_in = d < ds_end && 8 * d + wl_p < nblk;
#pragma unroll
      for (int i = 0; i < 8; ++i) sl.w[i] = buf_ld16(w_rs, w_in ? w_off[i] + 128u * d : kOutOfRange);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int b = 8 * d + 4 * u + g;
        const bool in = d < ds_end && b < nblk;
        sl.s[u] = __builtin_amdgcn_raw_buffer_load_b32(s_rs, (int)(in ? (uint32_t)b * N + s_col : kOutOfRange), 0, 0);
      }
    };
    auto load_a = [&](int q, MxA<MG>& da) {
      const int b = 4 * q + g;
      const bool in = q < 2 * ds_end && b < nblk;
#pragma unroll
      for (int qq = 0; qq < MG; ++qq)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          da.a[qq][t] = buf_ld16(a_rs, in ? a_off[qq] + (uint32_t)(32 * b + 8 * t) * 2u : kOutOfRange);
    };
    MxA<MG> a0, a1;
    // double step d: half step u = 0 uses a0 (and loads a1 with half step
    // 2d+1), u = 1 uses a1 (and loads a0 with 2d+2)
    auto step = [&](int d, const MxSlot& sl) {
      // stage the codes through the slab: other lanes read what a lane
      // writes, so the writes are fenced from the previous step's reads and
      // from this step's reads
      wave_lds_fence();
#pragma unroll
      for (int i = 0; i < 8; ++i) my_slab[w_dst[i]] = sl.w[i];
      wave_lds_fence();
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const MxA<MG>& ac = u == 0 ? a0 : a1;
        load_a(2 * d + u + 1, u == 0 ? a1 : a0);
        u32x4_t bw[kMxNJ];
#pragma unroll
        for (int j = 0; j < kMxNJ; ++j) bw[j] = my_slab[r_src[j][u]];
        float sc[kMxNJ];
#pragma unroll
        for (int j = 0; j < kMxNJ; ++j) sc[j] = ue8m0_to_f32((sl.s[u] >> (8 * j)) & 0xFF);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < kMxNJ; ++j) {
            const u32x4_t bq = dequant8(bw[j][t], sc[j]);
            acc[0][j] = mfma16x16x32(ac.a[0][t], bq, acc[0][j]);
            if (MG > 1 && nch > 1) {
#pragma unroll
              for (int qq = 1; qq < MG; ++qq) acc[qq][j] = mfma16x16x32(ac.a[qq][t], bq, acc[qq][j]);
            }
          }
      }
    };

    MxSlot s0, s1, s2;
    load(ds_begin, s0);
    load_a(2 * ds_begin, a0);
    load(ds_begin + 1, s1);
    int d = ds_begin;
    for (; d + 3 <= ds_end; d += 3) {
      load(d + 2, s2);
      step(d, s0);
      load(d + 3, s0);
      step(d + 1, s1);
      load(d + 4, s1);
      step(d + 2, s2);
    }
    // 0..2 double steps left; s0, s1 hold d, d+1 and a0 holds half step 2d
    if (d < ds_end) step(d, s0);
    if (d + 1 < ds_end) step(d + 1, s1);

    // Sum the four K partials (fixed order: wave 0, 1, 2, 3); wave w then
    // finishes accumulator element v = w (row 4g + w of each chunk) of all
    // four columns.
    float bb[kMxNJ];
    {
      // two 4-byte reads: the bias is only guaranteed 4-byte alignment
      const uint32_t* bp = reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + s_col);
      const uint32_t b01 = bp[0], b23 = bp[1];
      bb[0] = bf16lo(b01);
      bb[1] = bf16hi(b01);
      bb[2] = bf16lo(b23);
      bb[3] = bf16hi(b23);
    }
#pragma unroll
    for (int qq = 0; qq < MG; ++qq) {
      if (qq < nch) {
#pragma unroll
        for (int j = 0; j < kMxNJ; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[qq][j][v];
        __syncthreads();
        float sum[kMxNJ];
#pragma unroll
        for (int j = 0; j < kMxNJ; ++j) {
          float t = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < kMxWaves; ++w2) t += red[w2][j][wave][lane];
          sum[j] = t;
        }
        const int m = r0 + 16 * qq + 4 * g + wave;
        if (m < M && col_ok) {
          const size_t orow = (size_t)(row0 + m);
          if (GATE_UP) {
            const float h0 = clamped_glu(sum[0] + bb[0], sum[1] + bb[1]);
            const float h1 = clamped_glu(sum[2] + bb[2], sum[3] + bb[3]);
            *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + orow * (N / 2) + ncol / 2) =
                pack_bf16x2(h0, h1);
          } else {
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + orow * N + ncol) =
                f32x4_t{sum[0] + bb[0], sum[1] + bb[1], sum[2] + bb[2], sum[3] + bb[3]};
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
  const bool one = T * k <= kMxOneChunkMeanRows * E;
  auto kern = one ? gemv_mxfp4_kernel<GATE_UP, 1> : gemv_mxfp4_kernel<GATE_UP, 2>;
  hipLaunchKernelGGL(kern, grid, dim3(kMxWaves * kWave), 0, stream, (const bf16_t*)A, (const uint8_t*)Wq,
                     (const uint8_t*)Ws,
                     (const bf16_t*)bias, cnt, off, rows, K, N, GATE_UP ? k : 1, (int)a_rows, out);
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
