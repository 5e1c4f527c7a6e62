// FP8 W8A8 experts: the quantisers and the LDS-tiled MFMA grouped GEMMs.
//
// xserv "Phase 19: gpt-oss-20b MoE support", section 5 (FP8 W8A8: 8-bit
// weights with one scalar scale per expert, stored transposed [E][N][K]; one
// batched launch for all experts with the scales applied after the product),
// section 2 (gate_up GEMM -> bias -> clamped GLU, down GEMM -> bias) and
// section 4 (block-uniform early exits, masked tails).
//
// Format: OCP FP8 E4M3 (bias 7, largest finite 448, S.1111.111 NaN), the
// format the gfx950 f8f6f4 MFMAs read with format code 0.  A scale is
// s = amax / 448 and a code is E4M3(a * (448 / amax)), each in float32, with
// round-to-nearest-even and saturation at 448; amax = 0 takes s = 1.
// Weights have one scale per expert; activations one scale per row (a
// token's x row for gate_up, a (token, slot) row of h for down).  h is
// rounded to bf16 by the gate_up epilogue and quantised by the row kernel.
//
// Tiled GEMM: the bf16 kernel's (expert, m-tile) lookup, XCD-aware order and
// three-buffer token LDS ring (one barrier per step, at its start), with
// v_mfma_f32_16x16x128_f8f6f4 on K steps of 128 codes.  A workgroup covers
// 128 rows x 256 columns; each of its four waves 128 x 64 = 8 x 4 blocks of
// 16 x 16 (128 accumulators per lane).
//   K slots: operand byte q of lane group g (g = lane/16) is K = 64*(q/16) +
//   16g + q%16 of the step, for both operands, so the four lane groups' 16-byte
//   loads of a column or token row are one contiguous 64-byte run.
//   B (codes [E][N][K], K contiguous): lane (c = lane%16, g) of wave w loads,
//   for block j = 0..3, column n0 + 64w + 4c + j: two 16-byte loads a step,
//   issued back to back, which between them read the column's whole 128-byte
//   line (reading the line across two steps instead costs the L2 twice the
//   requests).  Two steps ahead, in a ring of three register sets.
//   A (codes of token rows): gathered through rows[] (gate_up) or contiguous
//   (down); each thread copies four 16-byte pieces a step, eight threads per
//   128-byte row, three steps ahead, into the fragment-major LDS ring two steps
//   ahead: fragment mi (rows 16mi..16mi+15) holds, in lane order, the 32
//   bytes lane l of the MFMA needs.  A step reads its fragments back two MFMA
//   groups before use into a ring of three: holding all eight fragments of a
//   step (64 registers) pushed the register allocator into rotating the
//   accumulators through spare registers every loop iteration, 72 moves each
//   waiting on an MFMA result.
// Epilogue: in the 16 x 16 accumulator layout lane l, element v holds row
// 4*(l/16) + v of MFMA column l%16, i.e. weight column n0 + 64w + 4c + j of
// block j: a lane holds two whole (gate, up) pairs.  Product * s_row *
// s_expert + bias, then GLU and one 4-byte bf16 h store (gate_up) or one
// 16-byte float32 store (down).
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace moe {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float kE4m3Max = 448.0f;

// float -> E4M3 code, nearest with ties to the even code, |v| >= 448 (and
// infinities) saturated to 448, NaN -> 0x7F.  With e = max(exponent, -6) the
// quantum of |v|'s binade is 2^(e-3), so q = rint(|v| * 2^(3-e)) (exact
// scaling, then round-half-even) is the value in quanta, and the code is
// (e + 6) * 8 + q: for normals that is ((e + 7) << 3) | (q - 8), below 2^-6 it
// is the subnormal code q, and q = 16 carries into the next binade's m = 0.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), kE4m3Max);
  const int e = max((int)(__float_as_uint(a) >> 23) - 127, -6);
  const uint32_t q = (uint32_t)__builtin_rintf(__builtin_amdgcn_ldexpf(a, 3 - e));
  const uint32_t code = sign | (uint32_t)((e + 6) * 8 + (int)q);
  return v != v ? 0x7Fu : code;
}

// (s, inv) of a float32 maximum: s = amax / 448, inv = 448 / amax, each
// rounded once; amax = 0 gives (1, 1).
__device__ __forceinline__ void fp8_scale(float amax, float& s, float& inv) {
  s = amax == 0.0f ? 1.0f : __fdiv_rn(amax, kE4m3Max);
  inv = amax == 0.0f ? 1.0f : __fdiv_rn(kE4m3Max, amax);
}

__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return a | (b << 8) | (c << 16) | (d << 24);
}

// eight bf16 (one 16-byte piece) * inv -> eight codes (8 bytes)
__device__ __forceinline__ u32x2_t encode8(u32x4_t v, float inv) {
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = e4m3_encode(bf16lo(v[i]) * inv);
    c[2 * i + 1] = e4m3_encode(bf16hi(v[i]) * inv);
  }
  return u32x2_t{pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7])};
}

// |bf16| maximum of a 16-byte piece, on the bit patterns (a NaN compares
// above every number, as in a NaN-propagating maximum)
__device__ __forceinline__ uint32_t absmax8(u32x4_t v) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(v[i] & 0x7FFFu, (v[i] >> 16) & 0x7FFFu));
  return m;
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// Row quantiser: one wave per row of K bf16 (K % 8 == 0): the row maximum,
// then the codes (the second pass re-reads the row from the cache).
// ---------------------------------------------------------------------------
constexpr int kRowWaves = 4;

// R_live (device, optional): rows from *R_live on are left untouched (the
// rows of h past the routed slots hold nothing and are never read).
__global__ __launch_bounds__(kRowWaves * kWave) void fp8_rows_kernel(const bf16_t* __restrict__ a, int64_t R, int K,
                                                                    const int32_t* __restrict__ R_live,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = (int64_t)blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  if (r >= R) return;                                    // wave-uniform, no barrier in this kernel
  if (R_live && r >= (int64_t)*R_live) return;           // wave-uniform
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a + r * K);
  const int nch = K / 8;
  uint32_t m = 0;
  for (int c = lane; c < nch; c += kWave) m = max(m, absmax8(src[c]));
  m = wave_max(m);
  float s, inv;
  fp8_scale(__uint_as_float(m << 16), s, inv);
  u32x2_t* dst = reinterpret_cast<u32x2_t*>(codes + r * K);
  for (int c = lane; c < nch; c += kWave) dst[c] = encode8(src[c], inv);
  if (lane == 0) scales[r] = s;
}

// ---------------------------------------------------------------------------
// Weight quantiser, W [E][K][N] bf16 -> codes [E][N][K], one scale per expert.
// 1. amax[e] = 0 (as bits); 2. atomic maximum of |bits| per expert (order
// free, so deterministic); 3. quantise and transpose 64 x 64 tiles through
// LDS; 4. amax -> scale in place.
// ---------------------------------------------------------------------------
__global__ void fp8_zero_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ __launch_bounds__(256) void fp8_amax_kernel(const bf16_t* __restrict__ W, int64_t per_expert,
                                                      uint32_t* __restrict__ amax) {
  const int e = blockIdx.y;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(W + (size_t)e * per_expert);
  const int64_t nch = per_expert / 8;
  uint32_t m = 0;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < nch; c += (int64_t)gridDim.x * blockDim.x)
    m = max(m, absmax8(src[c]));
  m = wave_max(m);
  if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(&amax[e], m << 16);
}

constexpr int kQt = 64;   // tile: 64 K x 64 N

__global__ __launch_bounds__(256) void fp8_weight_quant_kernel(const bf16_t* __restrict__ W, int K, int N,
                                                              const uint32_t* __restrict__ amax,
                                                              uint8_t* __restrict__ codes) {
  __shared__ float tile[kQt][kQt + 1];
  const int e = blockIdx.z;
  const int k0 = blockIdx.y * kQt, n0 = blockIdx.x * kQt;
  const int t = threadIdx.x;
  float s, inv;
  fp8_scale(__uint_as_float(amax[e]), s, inv);
  const bf16_t* We = W + (size_t)e * K * N;
  // load: thread t covers row k0 + t/8 (+32) and columns n0 + 8(t%8) .. +7
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = t / 8 + 32 * h, nc = 8 * (t % 8);
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (k0 + kr < K && n0 + nc < N) v = *reinterpret_cast<const u32x4_t*>(We + (size_t)(k0 + kr) * N + n0 + nc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[kr][nc + 2 * i] = bf16lo(v[i]);
      tile[kr][nc + 2 * i + 1] = bf16hi(v[i]);
    }
  }
  __syncthreads();
  // store: thread t writes column n0 + t/4, K codes k0 + 16(t%4) .. +15
  const int nc = t / 4, kc = 16 * (t % 4);
  if (n0 + nc < N && k0 + kc < K) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = pack4(e4m3_encode(tile[kc + 4 * q][nc] * inv), e4m3_encode(tile[kc + 4 * q + 1][nc] * inv),
                   e4m3_encode(tile[kc + 4 * q + 2][nc] * inv), e4m3_encode(tile[kc + 4 * q + 3][nc] * inv));
    *reinterpret_cast<u32x4_t*>(codes + ((size_t)e * N + n0 + nc) * K + k0 + kc) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

__global__ void fp8_scale_finalize_kernel(uint32_t* __restrict__ amax_to_scale, int E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  float s, inv;
  fp8_scale(__uint_as_float(amax_to_scale[e]), s, inv);
  amax_to_scale[e] = __float_as_uint(s);
}

// ---------------------------------------------------------------------------
// Tiled grouped GEMM
// ---------------------------------------------------------------------------
constexpr int kFgThreads = 256;
constexpr int kFgWaves = kFgThreads / kWave;
constexpr int kFgBM = 128;
constexpr int kFgWN = 64;
constexpr int kFgBN = kFgWaves * kFgWN;   // 256
constexpr int kFgBK = 128;                // codes per K step
constexpr int kFgLdsBufs = 3;
constexpr int kXcds = 8;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

struct FgSmem {
  u32x4_t a[kFgLdsBufs][kFgBM / 16][kWave][2];   // 3 x 8 fragments x 2 KB
  float srow[kFgBM];
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}
__device__ __forceinline__ f32x4_t mfma_fp8_16(const u32x4_t (&a)[2], const u32x4_t (&b)[2], f32x4_t c) {
  const i32x8_t av = {(int)a[0].x, (int)a[0].y, (int)a[0].z, (int)a[0].w,
                      (int)a[1].x, (int)a[1].y, (int)a[1].z, (int)a[1].w};
  const i32x8_t bv = {(int)b[0].x, (int)b[0].y, (int)b[0].z, (int)b[0].w,
                      (int)b[1].x, (int)b[1].y, (int)b[1].z, (int)b[1].w};
  // format 0 (E4M3) for both operands, no block scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
}

template <bool GATE_UP>
__global__ __launch_bounds__(kFgThreads, 1) void gemm_fp8_kernel(
    const uint8_t* __restrict__ A,        // gate_up: x codes [T][K]; down: h codes [S][K] (permuted order)
    const float* __restrict__ a_scale,    // gate_up: [T]; down: [S]
    const uint8_t* __restrict__ Wq,       // [E][N][K]
    const float* __restrict__ w_scale,    // [E]
    const bf16_t* __restrict__ bias,      // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,     // gate_up: permuted slot ids
    int K, int N, int E, int kslots, int a_rows, int n_tiles, int m_slots, void* __restrict__ out) {
  __shared__ __align__(16) FgSmem sm;
  __shared__ int s_tile[2];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  // ---- block -> (N tile, M-tile slot), consecutive slots on one XCD ----
  const int per_xcd = gridDim.x / kXcds;
  const int L = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (L >= n_tiles * m_slots) return;                       // block-uniform
  const int nt = L / m_slots;
  const int ms = L - nt * m_slots;

  // ---- M-tile slot -> (expert, first row) ----
  if (wave == 0) {
    if (lane == 0) s_tile[0] = -1;
    int tc[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane * 4 + i;
      tc[i] = e < E ? (cnt[e] + kFgBM - 1) / kFgBM : 0;
      sum += tc[i];
    }
    int start = wave_incl_scan(sum, lane) - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ms >= start && ms < start + tc[i]) {
        s_tile[0] = lane * 4 + i;
        s_tile[1] = (ms - start) * kFgBM;
      }
      start += tc[i];
    }
  }
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;                                         // block-uniform
  const int m0 = s_tile[1];
  const int M = cnt[e];
  const int row0 = off[e];
  const int n0 = nt * kFgBN;

  // ---- A: thread t copies pieces p = t + 256 s (s = 0..3) of the step: row
  // p/8 (rows past M read row M-1), 16 codes at K offset 16 (p%8); piece c8
  // belongs to lane group c8%4, operand half c8/4 of fragment row/16 ----
  const rsrc_t a_rs = make_rsrc(A, (uint32_t)((size_t)a_rows * K));
  const int a_c8 = tid & 7;
  uint32_t a_off[4];
  int a_dst[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int row = (tid >> 3) + 32 * s;
    const int m = min(m0 + row, M - 1);
    const uint32_t r = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
    a_off[s] = r * (uint32_t)K + 16u * a_c8;
    a_dst[s] = ((row >> 4) * kWave + (row & 15) + 16 * (a_c8 & 3)) * 2 + (a_c8 >> 2);
  }
  if (tid < kFgBM) {
    const int m = min(m0 + tid, M - 1);
    sm.srow[tid] = GATE_UP ? a_scale[rows[row0 + m] / kslots] : a_scale[row0 + m];
  }
  // ---- B: lane (c, g) of wave w, block j: column n0 + 64w + 4c + j ----
  const int g = lane >> 4;
  const int c = lane & 15;
  const int cw = n0 + wave * kFgWN + 4 * c;
  const rsrc_t w_rs = make_rsrc(Wq + (size_t)e * N * K, (uint32_t)N * (uint32_t)K);
  uint32_t b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) b_off[j] = (uint32_t)min(cw + j, N - 1) * (uint32_t)K + 16u * g;

  auto gload_a = [&](int kt, u32x4_t (&ra)[4]) {
    const uint32_t kb = (uint32_t)kt * kFgBK;
    const bool ok = (int)kb + 16 * a_c8 < K;
#pragma unroll
    for (int s = 0; s < 4; ++s) ra[s] = buf_ld16(a_rs, ok ? a_off[s] + kb : kOutOfRange);
  };
  auto gload_b = [&](int kt, u32x4_t (&rb)[4][2]) {
    const uint32_t kb = (uint32_t)kt * kFgBK;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool ok = (int)kb + 64 * h + 16 * g < K;
        rb[j][h] = buf_ld16(w_rs, ok ? b_off[j] + kb + 64u * h : kOutOfRange);
      }
  };
  u32x4_t* const lds_a = &sm.a[0][0][0][0];
  auto lstore = [&](int kt, const u32x4_t (&ra)[4]) {
    u32x4_t* const base = lds_a + (kt % kFgLdsBufs) * (kFgBM / 16) * kWave * 2;
#pragma unroll
    for (int s = 0; s < 4; ++s) base[a_dst[s]] = ra[s];
  };
  auto lread = [&](int buf, int mi, u32x4_t (&f)[2]) {
    f[0] = sm.a[buf][mi][lane][0];
    f[1] = sm.a[buf][mi][lane][1];
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mi][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Registers (the loop is unrolled three times and no ring needs a register
  // copy): B of steps kt, kt+1, kt+2 (Rb[kt%3] is used by step kt and then
  // reloaded, at step kt+1, with step kt+3); A of steps kt+2 and kt+3
  // (Ra[j%3] holds A(j) from its load, three steps ahead, to its LDS store,
  // two steps ahead); a ring of three A fragments (fragment mi of a step in
  // Fr[mi%3], read from LDS two groups before its MFMAs; the last two groups
  // of a step read fragments 0 and 1 of the next).
  u32x4_t Rb[3][4][2];
  u32x4_t Ra[3][4];
  u32x4_t Fr[3][2];

  // One K step kt (r = kt % 3): a barrier; issue the loads of A(kt+3), then
  // B(kt+2) (loads retire in order: a later store of A waits for A alone);
  // multiply B(kt) with the fragments of buffer kt%3; store A(kt+2) into
  // buffer (kt+2)%3 after the fourth group.  The barrier orders the previous
  // step's reads of buffer (kt+2)%3 before this store, and the previous
  // step's store into buffer (kt+1)%3 before this step's reads of it (its
  // last two groups read the next step's first fragments).
  auto step = [&](int kt, auto rc) {
    constexpr int r = decltype(rc)::value;
    const u32x4_t (&bt)[4][2] = Rb[r];
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    gload_a(kt + 3, Ra[r]);
    gload_b(kt + 2, Rb[(r + 2) % 3]);
    const int cbuf = kt % kFgLdsBufs, nbuf = (kt + 1) % kFgLdsBufs;
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      if (mi + 2 < 8) lread(cbuf, mi + 2, Fr[(mi + 2) % 3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mi][j] = mfma_fp8_16(Fr[mi % 3], bt[j], acc[mi][j]);
      if (mi == 3) lstore(kt + 2, Ra[(r + 2) % 3]);
      if (mi >= 6) lread(nbuf, mi - 6, Fr[mi % 3]);
    }
    // the twelve global loads over the first six groups; each fragment read
    // two groups ahead of its MFMAs
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      if (mi < 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // 1 MFMA
      if (mi < 6) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 global load
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (mi < 6) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (mi == 3) __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);  // 4 LDS writes
      if (mi >= 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Prologue: the loads in the order the steps issue them (A(j+3), then
  // B(j+2)), so the wait counts of the first steps match the later ones.
  const int nk = (K + kFgBK - 1) / kFgBK;
  gload_a(0, Ra[0]);
  gload_a(1, Ra[1]);
  gload_b(0, Rb[0]);
  lstore(0, Ra[0]);
  gload_a(2, Ra[2]);
  gload_b(1, Rb[1]);
  lstore(1, Ra[1]);
  __syncthreads();
  lread(0, 0, Fr[0]);
  lread(0, 1, Fr[1]);

  // The step count is rounded up to the unroll period: an extra step reads
  // only zeros (K past the end on both operands) and adds exactly 0.
  const int nk3 = (nk + 2) / 3 * 3;
  for (int kt = 0; kt < nk3; kt += 3) {
    step(kt + 0, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
    step(kt + 2, std::integral_constant<int, 2>{});
  }

  // ---- epilogue.  N % 4 == 0 and cw % 4 == 0: a lane's four columns are all
  // in range or all out of it. ----
  if (cw >= N) return;                                       // no barrier follows
  const float ws = w_scale[e];
  float bb[4];
  {
    const uint32_t* bp = reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + cw);
    const uint32_t b0 = bp[0], b1 = bp[1];
    bb[0] = bf16lo(b0);
    bb[1] = bf16hi(b0);
    bb[2] = bf16lo(b1);
    bb[3] = bf16hi(b1);
  }
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int rt = 16 * mi + 4 * g + v;   // row within the tile
      const int m = m0 + rt;
      if (m < M) {
        const float sc = sm.srow[rt] * ws;
        const size_t orow = (size_t)(row0 + m);
        if (GATE_UP) {
          const float h0 = clamped_glu(acc[mi][0][v] * sc + bb[0], acc[mi][1][v] * sc + bb[1]);
          const float h1 = clamped_glu(acc[mi][2][v] * sc + bb[2], acc[mi][3][v] * sc + bb[3]);
          *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + orow * (N / 2) + cw / 2) =
              pack_bf16x2(h0, h1);
        } else {
          *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + orow * N + cw) =
              f32x4_t{acc[mi][0][v] * sc + bb[0], acc[mi][1][v] * sc + bb[1], acc[mi][2][v] * sc + bb[2],
                      acc[mi][3][v] * sc + bb[3]};
        }
      }
    }
}

template <bool GATE_UP>
hipError_t launch_gemm(const void* A, const float* a_scale, const void* Wq, const float* w_scale, const void* bias,
                       const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int K, int N, int E,
                       int k, void* out, hipStream_t stream) {
  const int64_t S = T * k;
  const int64_t a_rows = GATE_UP ? T : S;
  // 32-bit buffer offsets: the token codes and one expert's codes below 2 GiB
  if (a_rows * K >= ((int64_t)1 << 31) || (int64_t)K * N >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  const int n_tiles = (N + kFgBN - 1) / kFgBN;
  const int64_t m_slots = (S + kFgBM - 1) / kFgBM + E;
  const int64_t blocks = (int64_t)n_tiles * m_slots;
  const int64_t grid = (blocks + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_fp8_kernel<GATE_UP>), dim3((unsigned)grid), dim3(kFgThreads), 0, stream,
                     (const uint8_t*)A, a_scale, (const uint8_t*)Wq, w_scale, (const bf16_t*)bias, cnt, off, rows, K,
                     N, E, k, (int)a_rows, n_tiles, (int)m_slots, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel (few rows per expert): a workgroup owns one expert
// and 64 output columns; its four waves split K and stream their part of the
// columns straight from HBM (no LDS staging), v_mfma_f32_16x16x128_f8f6f4 on
// K steps of 128 codes.  The four partial sums are added in LDS in a fixed
// order.
//   K slots: operand byte q of lane group g (g = lane/16) is K = 64*(q/16) +
//   16g + q%16 of the step, so lane (c = lane%16, g)'s two 16-byte pieces of
//   a column, together with the other three groups', read the column's 128
//   codes as two contiguous 64-byte runs.
//   Call j = 0..3 takes column n0 + 4c + j (a lane holds two whole (gate, up)
//   pairs); the token operand is 16 rows of x (or h) codes gathered in the
//   same K order, token rows (L2-resident) one step ahead.
//   Weight loads are line-coalesced instead (eight lanes per 128-byte line:
//   load i, lane L reads 16 codes of column 8i + L/8 at K offset 16 (L%8)),
//   two steps ahead in a ring of three register sets; each step writes its
//   set into the wave's own 8 KB LDS slab and reads back the MFMA operand
//   layout.  Slab address of (column, 16-byte piece p): column * 128 +
//   16 (p ^ ((column / 4) % 8)), which keeps the writes free of bank
//   conflicts and the operand reads at most two-way.
// ---------------------------------------------------------------------------
constexpr int kF8Waves = 4;
constexpr int kF8NJ = 4;                 // columns per lane
constexpr int kF8Cols = 16 * kF8NJ;      // 64 columns per workgroup
constexpr int kF8BK = 128;               // codes per K step

struct F8W {
  u32x4_t w[8];
};
template <int MG>
struct F8A {
  u32x4_t a[MG][2];
};

template <bool GATE_UP, int MG>
__global__ __launch_bounds__(kF8Waves * kWave) __attribute__((amdgpu_waves_per_eu(MG == 1 ? 2 : 1)))
void gemv_fp8_kernel(
    const uint8_t* __restrict__ A,        // gate_up: x codes [T][K]; down: h codes [S][K] (permuted order)
    const float* __restrict__ a_scale,    // gate_up: [T]; down: [S]
    const uint8_t* __restrict__ Wq,       // [E][N][K]
    const float* __restrict__ w_scale,    // [E]
    const bf16_t* __restrict__ bias,      // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,     // gate_up only: permuted slot ids
    int K, int N, int kslots, int a_rows, void* __restrict__ out) {
  __shared__ float red[kF8Waves][kF8NJ][4][kWave];   // 16 KB: one 16-row chunk's partial sums per wave
  __shared__ __align__(16) u32x4_t slab[kF8Waves][kF8Cols * 8];   // 32 KB: each wave's staged weight step

  const int e = blockIdx.y;
  const int M = cnt[e];
  if (M == 0) return;   // block-uniform: no load, no barrier for an expert without rows
  const int row0 = off[e];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4;
  const int c = lane & 15;
  // N % 4 == 0 and ncol % 4 == 0: a lane's four columns are all in range or all out
  const int ncol = blockIdx.x * kF8Cols + kF8NJ * c;
  const bool col_ok = ncol < N;

  const rsrc_t w_rs = make_rsrc(Wq + (size_t)e * N * K, (uint32_t)N * (uint32_t)K);
  const rsrc_t a_rs = make_rsrc(A, (uint32_t)((size_t)a_rows * K));
  // coalesced weight loads: load i covers slab columns 8i .. 8i+7
  const int wl_col = lane >> 3, wl_p = lane & 7;
  uint32_t w_off[8];
  int w_dst[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int col = 8 * i + wl_col;
    w_off[i] = (uint32_t)min(blockIdx.x * kF8Cols + col, N - 1) * (uint32_t)K + 16u * wl_p;
    w_dst[i] = col * 8 + (wl_p ^ ((col >> 2) & 7));
  }
  // operand reads: call j, half h of lane (c, g) = column 4c + j, piece 4h + g
  int r_src[kF8NJ][2];
#pragma unroll
  for (int j = 0; j < kF8NJ; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int col = 4 * c + j;
      r_src[j][h] = col * 8 + ((4 * h + g) ^ ((col >> 2) & 7));
    }
  u32x4_t* const my_slab = slab[wave];
  const int nk = (K + kF8BK - 1) / kF8BK;
  const int kb_begin = (nk * wave) / kF8Waves;
  const int kb_end = (nk * (wave + 1)) / kF8Waves;
  const float ws = w_scale[e];

  for (int r0 = 0; r0 < M; r0 += 16 * MG) {
    const int nch = min(MG, (M - r0 + 15) / 16);   // block-uniform
    uint32_t a_off[MG];
#pragma unroll
    for (int qq = 0; qq < MG; ++qq) {
      const int m = min(r0 + 16 * qq + c, M - 1);   // A row of this lane (clamped)
      const uint32_t r = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
      a_off[qq] = r * (uint32_t)K + 16u * g;
    }
    f32x4_t acc[MG][kF8NJ];
#pragma unroll
    for (int qq = 0; qq < MG; ++qq)
#pragma unroll
      for (int j = 0; j < kF8NJ; ++j) acc[qq][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // loads of step q; steps outside this wave's range and pieces past K
    // read 0 (sent outside the descriptors, no memory touched)
    auto load_w = [&](int q, F8W& d) {
      const uint32_t kb = (uint32_t)(q * kF8BK);
      const bool in = q < kb_end && (int)kb + 16 * wl_p < K;
#pragma unroll
      for (int i = 0; i < 8; ++i) d.w[i] = buf_ld16(w_rs, in ? w_off[i] + kb : kOutOfRange);
    };
    auto load_a = [&](int q, F8A<MG>& d) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t kb = (uint32_t)(q * kF8BK + 64 * h);
        const bool in = q < kb_end && (int)kb + 16 * g < K;
#pragma unroll
        for (int qq = 0; qq < MG; ++qq) d.a[qq][h] = buf_ld16(a_rs, in ? a_off[qq] + kb : kOutOfRange);
      }
    };
    auto step = [&](const F8W& dw, const F8A<MG>& da) {
      // stage through the slab: other lanes read what a lane writes, so the
      // writes are fenced from the previous step's reads and from this
      // step's reads
      wave_lds_fence();
#pragma unroll
      for (int i = 0; i < 8; ++i) my_slab[w_dst[i]] = dw.w[i];
      wave_lds_fence();
      u32x4_t bw[kF8NJ][2];
#pragma unroll
      for (int j = 0; j < kF8NJ; ++j) {
        bw[j][0] = my_slab[r_src[j][0]];
        bw[j][1] = my_slab[r_src[j][1]];
      }
#pragma unroll
      for (int j = 0; j < kF8NJ; ++j) {
        acc[0][j] = mfma_fp8_16(da.a[0], bw[j], acc[0][j]);
        if (MG > 1 && nch > 1) {
#pragma unroll
          for (int qq = 1; qq < MG; ++qq) acc[qq][j] = mfma_fp8_16(da.a[qq], bw[j], acc[qq][j]);
        }
      }
    };

    F8W w0, w1, w2;
    F8A<MG> a0, a1, a2;
    load_w(kb_begin, w0);
    load_w(kb_begin + 1, w1);
    load_a(kb_begin, a0);
    int q = kb_begin;
    for (; q + 3 <= kb_end; q += 3) {
      load_w(q + 2, w2);
      load_a(q + 1, a1);
      step(w0, a0);
      load_w(q + 3, w0);
      load_a(q + 2, a2);
      step(w1, a1);
      load_w(q + 4, w1);
      load_a(q + 3, a0);
      step(w2, a2);
    }
    // 0..2 steps left; w0, w1 hold steps q, q+1 and a0 holds step q
    if (q < kb_end) {
      load_a(q + 1, a1);
      step(w0, a0);
    }
    if (q + 1 < kb_end) step(w1, a1);

    // Sum the four K partials (fixed order: wave 0, 1, 2, 3); wave w then
    // finishes accumulator element v = w (row 4g + w of each chunk) of all
    // four columns.
    float bb[kF8NJ];
    {
      const uint32_t* bp = reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + min(ncol, N - kF8NJ));
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
        for (int j = 0; j < kF8NJ; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[wave][j][v][lane] = acc[qq][j][v];
        __syncthreads();
        float sum[kF8NJ];
#pragma unroll
        for (int j = 0; j < kF8NJ; ++j) {
          float t = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < kF8Waves; ++w2) t += red[w2][j][wave][lane];
          sum[j] = t;
        }
        const int m = r0 + 16 * qq + 4 * g + wave;
        if (m < M && col_ok) {
          const size_t orow = (size_t)(row0 + m);
          const float sc = (GATE_UP ? a_scale[rows[row0 + m] / kslots] : a_scale[orow]) * ws;
          if (GATE_UP) {
            const float h0 = clamped_glu(sum[0] * sc + bb[0], sum[1] * sc + bb[1]);
            const float h1 = clamped_glu(sum[2] * sc + bb[2], sum[3] * sc + bb[3]);
            *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(out) + orow * (N / 2) + ncol / 2) =
                pack_bf16x2(h0, h1);
          } else {
            *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(out) + orow * N + ncol) =
                f32x4_t{sum[0] * sc + bb[0], sum[1] * sc + bb[1], sum[2] * sc + bb[2], sum[3] * sc + bb[3]};
          }
        }
        __syncthreads();
      }
    }
  }
}

template <bool GATE_UP>
hipError_t launch_gemv(const void* A, const float* a_scale, const void* Wq, const float* w_scale, const void* bias,
                       const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int K, int N, int E,
                       int k, void* out, hipStream_t stream) {
  const int64_t S = T * k;
  const int64_t a_rows = GATE_UP ? T : S;
  if (a_rows * K >= ((int64_t)1 << 31) || (int64_t)K * N >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  const dim3 grid((N + kF8Cols - 1) / kF8Cols, E);
  // 32 rows per pass once the mean load per expert passes 10 rows
  const bool one = S <= 10 * (int64_t)E;
  auto kern = one ? gemv_fp8_kernel<GATE_UP, 1> : gemv_fp8_kernel<GATE_UP, 2>;
  hipLaunchKernelGGL(kern, grid, dim3(kF8Waves * kWave), 0, stream, (const uint8_t*)A, a_scale, (const uint8_t*)Wq, w_scale,
                     (const bf16_t*)bias, cnt, off, rows, K, N, GATE_UP ? k : 1, (int)a_rows, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize_rows(const void* a, int64_t R, int K, void* codes, float* scales, hipStream_t stream,
                                    const int32_t* R_live) {
  if (R == 0) return hipSuccess;
  const int64_t blocks = (R + kRowWaves - 1) / kRowWaves;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fp8_rows_kernel, dim3((unsigned)blocks), dim3(kRowWaves * kWave), 0, stream, (const bf16_t*)a, R,
                     K, R_live, (uint8_t*)codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_weights(const void* W, int E, int K, int N, void* codes, float* scales,
                                       hipStream_t stream) {
  uint32_t* amax = reinterpret_cast<uint32_t*>(scales);
  hipLaunchKernelGGL(fp8_zero_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, amax, E);
  const int64_t per_expert = (int64_t)K * N;
  const int64_t nch = per_expert / 8;
  const int gx = (int)std::min<int64_t>((nch + 255) / 256, 256);
  hipLaunchKernelGGL(fp8_amax_kernel, dim3(gx, E), dim3(256), 0, stream, (const bf16_t*)W, per_expert, amax);
  hipLaunchKernelGGL(fp8_weight_quant_kernel, dim3((N + kQt - 1) / kQt, (K + kQt - 1) / kQt, E), dim3(256), 0,
                     stream, (const bf16_t*)W, K, N, (const uint32_t*)amax, (uint8_t*)codes);
  hipLaunchKernelGGL(fp8_scale_finalize_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, amax, E);
  return hipGetLastError();
}

// The LDS-staged 256 x 256 kernel (fp8_gemm.hip) where K % 16 == 0, this
// kernel otherwise.
hipError_t launch_gemm_fp8_gate_up(const void* xq, const float* sx, const void* Wq, const float* Ws, const void* bgu,
                                   const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int H,
                                   int E, int k, int I, void* h, hipStream_t stream) {
  const hipError_t st = launch_gemm_fp8_lds_gate_up(xq, sx, Wq, Ws, bgu, cnt, off, rows, T, H, E, k, I, h, stream);
  if (st != hipErrorNotSupported) return st;
  return launch_gemm<true>(xq, sx, Wq, Ws, bgu, cnt, off, rows, T, H, 2 * I, E, k, h, stream);
}

hipError_t launch_gemm_fp8_down(const void* hq, const float* sh, const void* Wq, const float* Ws, const void* bd,
                                const int32_t* cnt, const int32_t* off, int64_t T, int H, int E, int k, int I,
                                float* o, hipStream_t stream) {
  const hipError_t st = launch_gemm_fp8_lds_down(hq, sh, Wq, Ws, bd, cnt, off, T, H, E, k, I, o, stream);
  if (st != hipErrorNotSupported) return st;
  return launch_gemm<false>(hq, sh, Wq, Ws, bd, cnt, off, nullptr, T, I, H, E, k, o, stream);
}

}  // namespace moe

namespace moe {
hipError_t launch_gemv_fp8_gate_up(const void* xq, const float* sx, const void* Wq, const float* Ws, const void* bgu,
                                   const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int H,
                                   int E, int k, int I, void* h, hipStream_t stream) {
  return launch_gemv<true>(xq, sx, Wq, Ws, bgu, cnt, off, rows, T, H, 2 * I, E, k, h, stream);
}

hipError_t launch_gemv_fp8_down(const void* hq, const float* sh, const void* Wq, const float* Ws, const void* bd,
                                const int32_t* cnt, const int32_t* off, int64_t T, int H, int E, int k, int I,
                                float* o, hipStream_t stream) {
  return launch_gemv<false>(hq, sh, Wq, Ws, bd, cnt, off, nullptr, T, I, H, E, k, o, stream);
}
}  // namespace moe
