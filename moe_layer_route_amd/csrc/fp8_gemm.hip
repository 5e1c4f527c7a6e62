// Tiled grouped GEMM of the FP8 W8A8 experts for large token counts per
// expert (the prefill regime, bound by the FP8 matrix cores and the load path).
//
// xserv "Phase 19: gpt-oss-20b MoE support": section 5 (8-bit weights with one
// scalar scale per expert, stored transposed [E][N][K], one batched launch and
// the scales applied after the product), section 2 (gate_up -> bias -> GLU,
// down -> bias), section 4 (early exits only when the whole workgroup leaves
// together; masked tails).
//
// Operands: token codes [rows][K] (x codes gathered through the permutation
// for gate_up, h codes in permuted order for down) with one float32 scale per
// row, and weight codes [E][N][K] with one scale per expert, both K
// contiguous.  Product in float32 on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3),
// then x s_row x s_expert + bias in the epilogue.
//
// Tile: 256 rows x 256 columns, K stages of 128 codes (one 128-byte line of
// every row), four waves in a 2 x 2 grid, each 128 x 128 = 4 x 4 blocks of
// 32 x 32 (256 float32 accumulators per lane).  A tile of this size moves 1/128
// byte per flop through the CU, half of what the same tile moves in bf16.
//   Staging: both operands HBM/L2 -> LDS by direct-to-LDS buffer loads
//   (buffer_load_dwordx4 ... lds, no register round trip), two stage buffers
//   of 64 KB.  One load instruction fills 1 KB = 8 rows x 128 bytes, eight
//   lanes per row, so every request is a whole cache line.  Row r's 16-byte
//   chunk c sits at slot c ^ ((r >> 1) & 7) of the row (conflict-free
//   fragment reads below); the load side realises it by which chunk each lane
//   fetches.  For gate_up the weight rows of a tile are taken in a regrouped
//   order: tile row 64q + 32s + t is weight row n0 + 2 (32q + t) + s, so the
//   gate and the up of a GLU pair land in the same lane of neighbouring
//   accumulator blocks.  Rows past the expert's count, columns past N and the
//   K tail are sent outside the buffer range and land as 0.
//   Fragments: a 32x32x64 operand is 32 rows x 64 codes: lane l holds row
//   l % 32, chunks 4j + 2 (l / 32) and 4j + 2 (l / 32) + 1 of step j (the same
//   K codes for both operands, which is all the product needs); two
//   ds_read_b128 per fragment.  Reads of step j are issued while the MFMAs of
//   step j - 1 run.
//   Stage s: after the barrier that ends stage s - 1, all loads of stage s+1
//   are issued into the other buffer (its reads ended before that barrier);
//   each wave waits for its own loads at the end of the stage and the barrier
//   makes all of them visible.
// Tile order: expert by expert; within an expert, each N tile's weight slab
// taken by all the expert's M tiles in turn (256-row tiles: a few per expert),
// consecutive tiles on one XCD (workgroup b runs on XCD b % 8).  Workgroups
// past the tile count exit before any load or barrier.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

#define LDS3 __attribute__((address_space(3)))

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kQgThreads = 256;
constexpr int kQgBM = 256;
constexpr int kQgBN = 256;
constexpr int kQgBK = 128;                              // codes per K stage
constexpr int kQgRowBytes = kQgBK;                      // 128
constexpr int kQgOpBytes = kQgBM * kQgRowBytes;         // 32 KB: one operand of one stage
constexpr int kQgA = 0;                                 // A of buffer b at b * 32 KB
constexpr int kQgB = 2 * kQgOpBytes;                    // B of buffer b at 64 KB + b * 32 KB
constexpr int kQgLds = 4 * kQgOpBytes;                  // 128 KB
constexpr int kQgMBlock = 1024;   // M tiles per block of the tile order: all of an expert's
constexpr int kXcds = 8;
constexpr uint32_t kQgOOR = 0x80000000u;               // beyond every descriptor's range

__device__ __forceinline__ f32x16_t mfma_fp8_32(const u32x4_t (&a)[2], const u32x4_t (&b)[2], f32x16_t c) {
  const i32x8_t av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                      (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
  const i32x8_t bv = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
                      (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
  // format 0 (E4M3) for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
}

template <bool GATE_UP>
__global__ __launch_bounds__(kQgThreads, 1) void gemm_fp8_lds_kernel(
    const uint8_t* __restrict__ A,        // gate_up: x codes [T][K]; down: h codes [S][K] (permuted order)
    const float* __restrict__ a_scale,    // gate_up: [T]; down: [S]
    const uint8_t* __restrict__ Wq,       // [E][N][K]
    const float* __restrict__ w_scale,    // [E]
    const bf16_t* __restrict__ bias,      // [E][N] (interleaved gate/up for gate_up)
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,     // gate_up: permuted slot ids
    int K, int N, int E, int kslots, int a_rows, int n_tiles, void* __restrict__ out) {
  __shared__ __align__(1024) char smem_g[kQgLds];
  LDS3 char* smem = (LDS3 char*)smem_g;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- workgroup -> (expert, M tile, N tile): the grouped tile order, every
  // wave finds the same ----
  int e, m0, nt;
  if (!grouped_gemm_tile(cnt, E, kQgBM, n_tiles, kQgMBlock, lane, e, m0, nt)) return;   // workgroup-uniform
  const int n0 = nt * kQgBN;
  const int M = cnt[e];
  const int row0 = off[e];
  const int ns = (K + kQgBK - 1) / kQgBK;

  // ---- direct-load assignments: wave w fills rows 64w .. 64w + 63 of both
  // tiles, eight rows per instruction; lane l takes row 8i + l / 8 of its
  // instruction i and chunk c = (l % 8) ^ ((r >> 1) & 7) of it ----
  const u32x4_t a_rs = rsrc_words(A, (uint32_t)((size_t)a_rows * K));
  const u32x4_t b_rs = rsrc_words(Wq + (size_t)e * N * K, (uint32_t)((size_t)N * K));
  const int lc[2] = {(lane & 7) ^ ((lane >> 4) & 7), (lane & 7) ^ (((lane >> 4) + 4) & 7)};  // even, odd i
  uint32_t a_off[8], b_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 64 * wave + 8 * i + (lane >> 3);
    const uint32_t c16 = 16u * (uint32_t)lc[i & 1];
    const int m = m0 + r;
    if (m < M) {
      const uint32_t tok = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
      a_off[i] = tok * (uint32_t)K + c16;
    } else {
      a_off[i] = kQgOOR;
    }
    const int n = GATE_UP ? n0 + (r & ~63) + 2 * (r & 31) + ((r >> 5) & 1) : n0 + r;
    b_off[i] = n < N ? (uint32_t)n * (uint32_t)K + c16 : kQgOOR;
  }
  // A lane's chunk is past K when k0 >= K - 16 c (K % 16 == 0: a chunk is all
  // in or all out); such loads and those of stages past the last one go
  // outside the range.  The vector offset carries the row, the scalar offset
  // the K stage.
  const int klim[2] = {K - 16 * lc[0], K - 16 * lc[1]};
  auto dma = [&](int st, int buf, int i, bool b_side) {
    const int k0 = st * kQgBK;
    const uint32_t base = b_side ? b_off[i] : a_off[i];
    const uint32_t voff = k0 < klim[i & 1] ? base : kQgOOR;
    const uint32_t lds = lds0 + (b_side ? kQgB : kQgA) + buf * kQgOpBytes + (64 * wave + 8 * i) * kQgRowBytes;
    dma16(b_side ? b_rs : a_rs, voff, (uint32_t)k0, lds);
  };

  // ---- fragment reads: step j (codes 64j .. 64j + 63 of the stage) ----
  const int fr = lane & 31;
  const int fg = lane >> 5;
  uint32_t a_rd[2][2], b_rd[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t xo = 16u * (uint32_t)((4 * j + 2 * fg + h) ^ ((fr >> 1) & 7));
      a_rd[j][h] = (uint32_t)(kQgA + (128 * wm + fr) * kQgRowBytes) + xo;
      b_rd[j][h] = (uint32_t)(kQgB + (128 * wn + fr) * kQgRowBytes) + xo;
    }
  auto read_frag = [&](int buf, int j, int q, bool b_side, u32x4_t (&f)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      f[h] = *(const LDS3 u32x4_t*)(smem + (b_side ? b_rd[j][h] : a_rd[j][h]) + buf * kQgOpBytes +
                                    q * 32 * kQgRowBytes);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // MFMA order of a step: the fragments in the order they are read (a0 b0
  // a1 b1 ...), each product as soon as both its operands are there.
  constexpr int kOrd[16][2] = {{0, 0}, {0, 1}, {1, 0}, {1, 1}, {0, 2}, {1, 2}, {2, 0}, {2, 1},
                               {2, 2}, {0, 3}, {1, 3}, {2, 3}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};
  auto mfma_at = [&](int t, const u32x4_t (&fa)[4][2], const u32x4_t (&fb)[4][2]) {
    const int i = kOrd[t][0], j = kOrd[t][1];
    acc[i][j] = mfma_fp8_32(fa[i], fb[j], acc[i][j]);
  };

  // prologue: stage 0 into buffer 0
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    dma(0, 0, i, false);
    dma(0, 0, i, true);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();

  u32x4_t fa0[4][2], fb0[4][2], fa1[4][2], fb1[4][2];
  // One half q of stage s (K step q) in four slots: slot u reads fragments u
  // of both operands for step q and issues four MFMAs of the previous step;
  // in the first half, each slot also issues four loads of stage s + 1 (a
  // stage past the last one is past K and loads nothing).
  auto half_stage = [&](int s, int buf, int q, u32x4_t (&fa_rd)[4][2], u32x4_t (&fb_rd)[4][2],
                        const u32x4_t (&fa_mm)[4][2], const u32x4_t (&fb_mm)[4][2], bool do_mfma) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (q == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dma(s + 1, buf ^ 1, 2 * u + (i >> 1), (i & 1) != 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      read_frag(buf, q, u, false, fa_rd[u]);
      read_frag(buf, q, u, true, fb_rd[u]);
      if (do_mfma) {
#pragma unroll
        for (int t = 4 * u; t < 4 * u + 4; ++t) mfma_at(t, fa_mm, fb_mm);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // two MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int s = 0; s < ns; ++s) {
    const int buf = s & 1;
    half_stage(s, buf, 0, fa0, fb0, fa1, fb1, s > 0);
    half_stage(s, buf, 1, fa1, fb1, fa0, fb0, true);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
  }
#pragma unroll
  for (int t = 0; t < 16; ++t) mfma_at(t, fa1, fb1);

  // ---- epilogue: the tile's row scales through LDS (the stage buffers are
  // free after the last barrier), then scale, bias and GLU or float32 o ----
  float* s_row = (float*)smem_g;
  {
    const int m = m0 + tid;
    float sr = 0.f;
    if (m < M) sr = a_scale[GATE_UP ? rows[row0 + m] / kslots : row0 + m];
    s_row[tid] = sr;
  }
  __syncthreads();
  const float ws = w_scale[e];
  const int half = lane >> 5;
  if (GATE_UP) {
    const int I = N / 2;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int P = (n0 + 128 * wn) / 2 + 32 * p + fr;
      if (P >= I) continue;
      const uint32_t bw = *reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + 2 * P);
      const float bg = bf16lo(bw), bu = bf16hi(bw);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rt = 128 * wm + 32 * rb + 8 * (v >> 2) + 4 * half + (v & 3);
          const int m = m0 + rt;
          if (m < M) {
            const float sc = s_row[rt] * ws;
            const float hv = clamped_glu(acc[rb][2 * p][v] * sc + bg, acc[rb][2 * p + 1][v] * sc + bu);
            reinterpret_cast<uint16_t*>(out)[(size_t)(row0 + m) * I + P] = (uint16_t)f32_to_bf16(hv);
          }
        }
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int n = n0 + 128 * wn + 32 * cb + fr;
      if (n >= N) continue;
      const float bb = bf16_to_f32(bias[(size_t)e * N + n]);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rt = 128 * wm + 32 * rb + 8 * (v >> 2) + 4 * half + (v & 3);
          const int m = m0 + rt;
          if (m < M)
            reinterpret_cast<float*>(out)[(size_t)(row0 + m) * N + n] = acc[rb][cb][v] * (s_row[rt] * ws) + bb;
        }
    }
  }
}

template <bool GATE_UP>
hipError_t launch(const void* A, const float* a_scale, const void* Wq, const float* w_scale, const void* bias,
                  const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int K, int N, int E, int k,
                  void* out, hipStream_t stream) {
  const int64_t S = T * k;
  const int64_t a_rows = GATE_UP ? T : S;
  if (K % 16 != 0 || (GATE_UP && N % 64 != 0)) return hipErrorNotSupported;
  // 32-bit buffer offsets: the token codes and one expert's codes below 2 GiB
  if (a_rows * K >= ((int64_t)1 << 31) || (int64_t)K * N >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  const int n_tiles = (N + kQgBN - 1) / kQgBN;
  // at most sum_e ceil(cnt_e / BM) <= S / BM + min(E, S) M tiles
  const int64_t tiles = (S / kQgBM + (S < E ? S : E)) * n_tiles;
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_fp8_lds_kernel<GATE_UP>), dim3((unsigned)grid), dim3(kQgThreads), 0, stream,
                     (const uint8_t*)A, a_scale, (const uint8_t*)Wq, w_scale, (const bf16_t*)bias, cnt, off, rows,
                     K, N, E, k, (int)a_rows, n_tiles, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8_lds_gate_up(const void* xq, const float* sx, const void* Wq, const float* Ws,
                                       const void* bgu, const int32_t* cnt, const int32_t* off, const int32_t* rows,
                                       int64_t T, int H, int E, int k, int I, void* h, hipStream_t stream) {
  return launch<true>(xq, sx, Wq, Ws, bgu, cnt, off, rows, T, H, 2 * I, E, k, h, stream);
}

hipError_t launch_gemm_fp8_lds_down(const void* hq, const float* sh, const void* Wq, const float* Ws, const void* bd,
                                    const int32_t* cnt, const int32_t* off, int64_t T, int H, int E, int k, int I,
                                    float* o, hipStream_t stream) {
  return launch<false>(hq, sh, Wq, Ws, bd, cnt, off, nullptr, T, I, H, E, k, o, stream);
}

}  // namespace moe
