// LDS-tiled MFMA grouped GEMMs of the experts with MXFP4 weights (large token
// counts per expert).
//
// xserv "Phase 19: gpt-oss-20b MoE support": section 5 (MXFP4 W4A16: E2M1
// weights with one UE8M0 scale per 32 values, bf16 activations), section 2
// (per-expert gate_up GEMM -> bias -> clamped GLU, down GEMM -> bias),
// section 5 (one batched launch for all experts) and section 4 (early exits
// only when the whole workgroup leaves together; masked tails).
//
// The tiling, the tile order, the token-row LDS ring and the epilogue are
// those of the bf16 grouped GEMM (gemm.hip): 128 x 512 tiles, four waves (one
// per SIMD) of 128 x 128, 8 x 8 tiles of v_mfma_f32_16x16x32_bf16 with the
// accumulators in the AGPRs.  What changes is the weight operand:
//   the codes are K-contiguous ([E][N][K/2]), so lane (g = lane/16,
//   c = lane%16) of wave w reads block 4q+g of columns cw+j (cw = n0 + 128w +
//   8c, j = 0..7) once per quad q of four 32-value blocks (128 K): eight
//   16-byte loads, plus the eight columns' scales of that block in one 8-byte
//   load (scales are block-major, [E][K/32][N]).  The quad's four 32-K MFMA
//   steps t use quarter t of each block: v_cvt_scalef32_pk_bf16_fp4 turns its
//   dword into the eight-value B operand of call j (MFMA column c of call j =
//   weight column cw + j, as in the bf16 kernel) -- no transpose.  (Loading
//   a quarter per step instead costs four times the L1 and L2 requests for
//   the same bytes, and the kernel then waits on them.)
//   The MFMA K slot (g, i) of step (q, t) is K = 128q + 32g + 8t + i, so the
//   token rows are gathered in that order: lane (row, g) copies the 16 bytes
//   of x at K = 128q + 32g + 8t.
//   Past the end of K the token loads return zeros; the weight loads there are
//   not masked (they read codes of the next column, or zeros past the last),
//   which is harmless since E2M1 codes are finite and scales past the last
//   block read as 0 (2^-127): those products are exactly zero.
#include "device_common.h"
#include "launch.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kMgThreads = 256;
constexpr int kMgWaves = kMgThreads / kWave;
constexpr int kMgBM = 128;
constexpr int kMgWN = 128;                    // columns per wave
constexpr int kMgBN = kMgWaves * kMgWN;       // 512
constexpr int kMgLdsBufs = 3;
constexpr int kXcds = 8;
constexpr int kMgMBlock = 8;   // M tiles per block of the tile order
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // a voffset no descriptor here reaches

struct MgSmem {
  u32x4_t a[kMgLdsBufs][kMgBM / 16][kWave];   // 3 x 8 fragments x 1 KB
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
// UE8M0 byte s -> float32 scale 2^(s - 127), in three VALU operations:
// 2^-127 * 2^s is exact for every s (2^-127 itself is a float32 subnormal,
// which the kernel's float mode keeps); s = 255 overflows to +inf, and
// fma(inf, 0, inf) turns that into NaN while leaving every finite scale as is.
__device__ __forceinline__ float ue8m0_f32(uint32_t word, int byte) {
  const int s = (int)__builtin_amdgcn_ubfe(word, 8 * byte, 8);
  const float f = __builtin_amdgcn_ldexpf(__uint_as_float(0x00400000u), s);
  return __builtin_fmaf(f, 0.0f, f);
}
// eight E2M1 codes (one dword, k = 0..7 from the low nibble up) -> eight bf16 * scale
__device__ __forceinline__ u32x4_t fp4x8_to_bf16(uint32_t w, float s) {
  const bf16x2_v a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0);
  const bf16x2_v b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1);
  const bf16x2_v c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2);
  const bf16x2_v d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3);
  return u32x4_t{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, c),
                 __builtin_bit_cast(uint32_t, d)};
}

template <bool GATE_UP>
__global__ __launch_bounds__(kMgThreads, 1) void gemm_mxfp4_kernel(
    const bf16_t* __restrict__ A,      // gate_up: x [T][K]; down: h [S][K] (permuted order)
    const uint8_t* __restrict__ Wq,    // [E][N][K/2]
    const uint8_t* __restrict__ Ws,    // [E][K/32][N]
    const bf16_t* __restrict__ bias,   // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,  // gate_up: permuted slot ids
    int K, int N, int E, int kslots, int a_rows, int n_tiles, void* __restrict__ out) {
  __shared__ __align__(16) MgSmem sm;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  // ---- block -> (expert, M tile, N tile): the grouped tile order.  Wave 0
  // finds it and hands it over through LDS (the lookup's registers, live in
  // every wave, would push this kernel's accumulator-bound allocation into
  // spills) ----
  __shared__ int s_tile[3];
  if (wave == 0) {
    int te, tm, tn;
    const bool ok = grouped_gemm_tile(cnt, E, kMgBM, n_tiles, kMgMBlock, lane, te, tm, tn);
    if (lane == 0) {
      s_tile[0] = ok ? te : -1;
      s_tile[1] = tm;
      s_tile[2] = tn;
    }
  }
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;                                         // block-uniform
  const int m0 = s_tile[1];
  const int nt = s_tile[2];
  const int M = cnt[e];
  const int row0 = off[e];
  const int n0 = nt * kMgBN;
  const int nblk = K / 32;

  // ---- global load assignments (unconditional buffer loads; rows past M
  // and columns past N read a valid row or column, K past the end reads 0) ----
  // A: thread (wave w, lane l) copies lane l of fragments w and w + 4: row
  // 16 f + l%16, the 8 values at K = 128q + 32 (l/16) + 8t of step (q, t)
  const rsrc_t a_rs = make_rsrc(A, (uint32_t)((size_t)a_rows * K * 2));
  const int a_kc = lane >> 4;
  uint32_t a_off[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int m = min(m0 + 16 * (wave + kMgWaves * s) + (lane & 15), M - 1);
    const uint32_t r = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
    a_off[s] = (r * (uint32_t)K + 32u * a_kc) * 2u;
  }
  // B: lane (g, c) of wave w reads block 4q+g of columns cw .. cw+7
  const int g = lane >> 4;
  const int c = lane & 15;
  const int cw = n0 + wave * kMgWN + 8 * c;
  const uint32_t row_bytes = (uint32_t)K / 2;
  const rsrc_t w_rs = make_rsrc(Wq + (size_t)e * N * row_bytes, (uint32_t)N * row_bytes);
  const rsrc_t s_rs = make_rsrc(Ws + (size_t)e * nblk * N, (uint32_t)(nblk * N));
  const uint32_t w_col = (uint32_t)min(cw, N - 8);
  const uint32_t w_lane = w_col * row_bytes + 16u * (uint32_t)g;
  const uint32_t s_lane = (uint32_t)g * N + w_col;

  // the codes and scales of quad q (whole offsets in the VGPR operand,
  // which the descriptor's range check covers)
  auto gload_q = [&](int q, u32x4_t (&wq)[8], u32x2_t& sq) {
    const uint32_t wo = w_lane + 64u * (uint32_t)q;
#pragma unroll
    for (int j = 0; j < 8; ++j) wq[j] = buf_ld16(w_rs, wo + (uint32_t)j * row_bytes);
    sq = __builtin_bit_cast(u32x2_t,
                            __builtin_amdgcn_raw_buffer_load_b64(s_rs, (int)(s_lane + 4u * (uint32_t)q * N), 0, 0));
  };
  auto gload_a = [&](int kt, u32x4_t (&ra)[2]) {
    const int q = kt >> 2, t = kt & 3;
    const int kidx = 128 * q + 32 * a_kc + 8 * t;
    const bool ok = kidx < K;
    const uint32_t kb = (uint32_t)(128 * q + 8 * t) * 2u;
#pragma unroll
    for (int s = 0; s < 2; ++s) ra[s] = buf_ld16(a_rs, ok ? a_off[s] + kb : kOutOfRange);
  };
  auto lstore = [&](int kt, const u32x4_t (&ra)[2]) {
    const int buf = kt % kMgLdsBufs;
    sm.a[buf][wave][lane] = ra[0];
    sm.a[buf][wave + kMgWaves][lane] = ra[1];
  };

  f32x4_t acc[8][8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mi][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Registers: the codes and scales of quad q (Q, S; S decoded into sc at
  // the quad's first step) and of quad q+1 (Qn, Sn: loaded at the quad's
  // first step, copied into Q and S after its last), A of steps kt+2 and
  // kt+3, and the A fragments F of step kt (each reloaded with step kt+1
  // after its last MFMA).
  u32x4_t Q[8], Qn[8];
  u32x2_t S, Sn;
  float sc[8];
  u32x4_t Ra0[2], Ra1[2];
  u32x4_t F[8];

  // One 32-K step kt = 4q + t: dequantise quarter t of the quad's codes;
  // issue the loads of A(kt+3) and (at t = 0) of quad q+1 -- in that order,
  // so that the store of A(kt+3) at the next step does not wait for the
  // quad's codes, as loads retire in order -- multiply while
  // reading the A fragments of kt+1 from LDS; store A(kt+2); one barrier
  // after the fifth of the eight MFMA groups.  The LDS ring and the
  // scheduling fences are those of the bf16 kernel: buffer (kt+1)%3 is read
  // during step kt and buffer (kt+2)%3 written before its barrier; the
  // global loads are spread over the MFMAs before the barrier.  Each step is
  // fenced off from its neighbours.
  auto step = [&](int q, auto tc, u32x4_t (&ra_load)[2], const u32x4_t (&ra_store)[2]) {
    constexpr int t = decltype(tc)::value;
    const int kt = 4 * q + t;
    __builtin_amdgcn_sched_barrier(0);
    if (t == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sc[j] = ue8m0_f32(j < 4 ? S.x : S.y, j & 3);
    }
    u32x4_t bt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bt[j] = fp4x8_to_bf16(Q[j][t], sc[j]);
    asm volatile("" ::"v"(bt[0]), "v"(bt[1]), "v"(bt[2]), "v"(bt[3]), "v"(bt[4]), "v"(bt[5]), "v"(bt[6]),
                 "v"(bt[7])
                 : "memory");
    __builtin_amdgcn_sched_barrier(0);
    gload_a(kt + 3, ra_load);
    if (t == 0) gload_q(q + 1, Qn, Sn);
    const int nbuf = (kt + 1) % kMgLdsBufs;
    auto group = [&](int mi) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[mi][j] = mfma16x16x32(F[mi], bt[j], acc[mi][j]);
    };
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      group(mi);
      F[mi] = sm.a[nbuf][mi][lane];
    }
    lstore(kt + 2, ra_store);
    group(4);
    if (t == 0) {   // eleven loads
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 global load
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);     // 2 LDS writes
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    } else {        // the two loads of A
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (mi < 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    __syncthreads();
    F[4] = sm.a[nbuf][4][lane];
#pragma unroll
    for (int mi = 5; mi < 8; ++mi) {
      group(mi);
      F[mi] = sm.a[nbuf][mi][lane];
    }
    if (t == 3) {
#pragma unroll
      for (int j = 0; j < 8; ++j) Q[j] = Qn[j];
      S = Sn;
    }
  };

  // Prologue: quad 0's codes and scales, A(0..2) (A(0), A(1) stored in
  // LDS).
  const int nq = (nblk + 3) / 4;
  gload_q(0, Q, S);
  gload_a(0, Ra0);
  gload_a(1, Ra1);
  lstore(0, Ra0);
  gload_a(2, Ra0);
  lstore(1, Ra1);
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) F[mi] = sm.a[0][mi][lane];

  // the A ring parity is the same at every quad start (four steps a quad)
  for (int q = 0; q < nq; ++q) {
    step(q, std::integral_constant<int, 0>{}, Ra1, Ra0);
    step(q, std::integral_constant<int, 1>{}, Ra0, Ra1);
    step(q, std::integral_constant<int, 2>{}, Ra1, Ra0);
    step(q, std::integral_constant<int, 3>{}, Ra0, Ra1);
  }

  // ---- epilogue (the bf16 kernel's).  16x16 accumulator layout: lane l,
  // element v holds row 4*(l/16) + v of MFMA column l%16 = weight column
  // cw + j of call j.  N % 8 == 0 and cw % 8 == 0: a lane's eight columns are
  // all in range or all out of it.
  if (cw >= N) return;                                       // no barrier follows
  float bb[8];
  {
    const uint32_t* bp = reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + cw);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const uint32_t bw = bp[qq];
      bb[2 * qq] = bf16lo(bw);
      bb[2 * qq + 1] = bf16hi(bw);
    }
  }
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + mi * 16 + 4 * g + v;
      if (m < M) {
        const size_t orow = (size_t)(row0 + m);
        if (GATE_UP) {
          uint32_t hw[2];
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const float h0 = clamped_glu(acc[mi][4 * qq][v] + bb[4 * qq], acc[mi][4 * qq + 1][v] + bb[4 * qq + 1]);
            const float h1 =
                clamped_glu(acc[mi][4 * qq + 2][v] + bb[4 * qq + 2], acc[mi][4 * qq + 3][v] + bb[4 * qq + 3]);
            hw[qq] = pack_bf16x2(h0, h1);
          }
          *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(out) + orow * (N / 2) + cw / 2) =
              u32x2_t{hw[0], hw[1]};
        } else {
          float* op = reinterpret_cast<float*>(out) + orow * N + cw;
          *reinterpret_cast<f32x4_t*>(op) = f32x4_t{acc[mi][0][v] + bb[0], acc[mi][1][v] + bb[1],
                                                    acc[mi][2][v] + bb[2], acc[mi][3][v] + bb[3]};
          *reinterpret_cast<f32x4_t*>(op + 4) = f32x4_t{acc[mi][4][v] + bb[4], acc[mi][5][v] + bb[5],
                                                        acc[mi][6][v] + bb[6], acc[mi][7][v] + bb[7]};
        }
      }
    }
}

template <bool GATE_UP>
hipError_t launch(const void* A, const void* Wq, const void* Ws, const void* bias, const int32_t* cnt,
                  const int32_t* off, const int32_t* rows, int64_t T, int K, int N, int E, int k, void* out,
                  hipStream_t stream) {
  const int64_t S = T * k;
  const int64_t a_rows = GATE_UP ? T : S;
  // 32-bit buffer offsets: the token operand and one expert's codes below
  // 2 GiB, so no in-range offset comes near kOutOfRange
  if (a_rows * K * 2 >= ((int64_t)1 << 31) || (int64_t)K * N / 2 >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  const int n_tiles = (N + kMgBN - 1) / kMgBN;
  const int64_t m_slots = (S + kMgBM - 1) / kMgBM + E;
  const int64_t blocks = (int64_t)n_tiles * m_slots;
  const int64_t grid = (blocks + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_mxfp4_kernel<GATE_UP>), dim3((unsigned)grid), dim3(kMgThreads), 0, stream,
                     (const bf16_t*)A, (const uint8_t*)Wq, (const uint8_t*)Ws, (const bf16_t*)bias, cnt, off, rows,
                     K, N, E, k, (int)a_rows, n_tiles, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mxfp4_gate_up(const void* x, const void* Wq, const void* Ws, const void* bgu,
                                     const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int H,
                                     int E, int k, int I, void* h, hipStream_t stream) {
  return launch<true>(x, Wq, Ws, bgu, cnt, off, rows, T, H, 2 * I, E, k, h, stream);
}

hipError_t launch_gemm_mxfp4_down(const void* h, const void* Wq, const void* Ws, const void* bd, const int32_t* cnt,
                                  const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                                  hipStream_t stream) {
  return launch<false>(h, Wq, Ws, bd, cnt, off, nullptr, T, I, H, E, k, o, stream);
}

}  // namespace moe
