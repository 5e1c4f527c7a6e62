// LDS-tiled MFMA grouped GEMMs of the experts (large token counts per expert).
//
// xserv "Phase 19: gpt-oss-20b MoE support": section 2 (per-expert gate_up GEMM
// -> bias -> clamped GLU, per-expert down GEMM -> bias), section 5 (one
// batched launch for all experts instead of one small GEMM per expert) and
// section 4 (early exits only when the whole workgroup leaves together;
// masked tails because N = 2880 is not a multiple of 128).
//
// One launch covers every expert.  The grid is sized from host-known T, k, E
// only: (number of N tiles) x (an upper bound on the M tiles of all experts,
// ceil(T*k / BM) + E).  Each workgroup finds its (expert, M tile, N tile) from
// cnt[] (prefix sum of ceil(cnt[e] / BM) x N tiles); surplus blocks exit before
// any load or barrier.  Tiles go expert by expert, in blocks of at most eight M
// tiles that take each N tile's weight slab in turn, and consecutive tiles run
// on one XCD, whose L2 serves both reuses.
//
// Tile: 128 rows x 512 columns, K steps of 32, four waves (one per SIMD) side
// by side along N.  Each wave owns 128 rows x 128 columns = 8 x 8 tiles of
// v_mfma_f32_16x16x32_bf16 (256 fp32 accumulators per lane, which live in the
// accumulation registers: one wave per SIMD has the whole register file).
//   B (weight, [K][N] with N contiguous): no two waves share a column, so B
//     bypasses LDS.  Lane (g = lane/16, c = lane%16) loads rows k0+8g ..
//     k0+8g+7 of the 8 columns c0+8c .. c0+8c+7 (eight 16-byte buffer loads,
//     two K steps ahead); an 8x8 transpose in registers turns them into
//     eight K-packed B operands: operand j holds column c0+8c+j in MFMA
//     column c.
//   A (token rows, k contiguous) is shared by the four waves: gathered
//     through rows[] (gate_up) or contiguous rows of h (down), loaded into
//     registers three K steps ahead, stored into a ring of three LDS buffers
//     two steps ahead, and read back into registers one step ahead (each
//     fragment as soon as its last MFMA of the current step has issued), so
//     the MFMAs of a step never wait on LDS.  The buffers are fragment-major:
//     fragment mi (rows 16 mi .. 16 mi + 15) is 1 KB holding, in lane order,
//     the 16 bytes lane l of the MFMA needs (row l%16, k chunk l/16), so
//     every fragment read and every store is one contiguous 1 KB access,
//     free of bank conflicts.  One barrier per K step.
// Epilogue: in the 16x16 accumulator layout lane l holds rows 4*(l/16)+0..3
// of MFMA column l%16, i.e. weight columns c0+8c+j of operands j = 0..7, so
// gate (j even) and up (j+1) of one pair sit in the same lane: bias + clamped
// GLU in registers, four h values stored as one 8-byte bf16 write (gate_up);
// bias and two 16-byte float32 writes (down).
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kGmThreads = 256;
constexpr int kGmWaves = kGmThreads / kWave;
constexpr int kGmBM = 128;
constexpr int kGmWN = 128;                    // columns per wave
constexpr int kGmBN = kGmWaves * kGmWN;       // 512
constexpr int kGmBK = 32;
constexpr int kGmLdsBufs = 3;
constexpr int kXcds = 8;
constexpr int kGmMBlock = 8;   // M tiles per block of the tile order
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // a voffset no descriptor here reaches

struct GemmSmem {
  u32x4_t a[kGmLdsBufs][kGmBM / 16][kWave];   // 3 x 8 fragments x 1 KB
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over [base, base + bytes): loads whose vector offset
// reaches past the end return 0 without touching memory.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

template <bool GATE_UP>
__global__ __launch_bounds__(kGmThreads, 1) void gemm_expert_kernel(
    const bf16_t* __restrict__ A,      // gate_up: x [T][K]; down: h [S][K] (permuted order)
    const bf16_t* __restrict__ W,      // [E][K][N]
    const bf16_t* __restrict__ bias,   // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,  // gate_up: permuted slot ids
    int K, int N, int E, int kslots, int a_rows, int n_tiles, void* __restrict__ out) {
  __shared__ __align__(16) GemmSmem sm;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave-uniform, stated so: it selects LDS fragments and weight columns
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  // ---- block -> (expert, M tile, N tile): the grouped tile order, every wave
  // finds the same ----
  int e, m0, nt;
  if (!grouped_gemm_tile(cnt, E, kGmBM, n_tiles, kGmMBlock, lane, e, m0, nt)) return;   // block-uniform
  const int M = cnt[e];
  const int row0 = off[e];
  const int n0 = nt * kGmBN;

  // ---- global load assignments ----
  // Every load is an unconditional buffer load (a masked load becomes a
  // branch, and the compiler then drains all outstanding loads at the merge).
  // Rows past M and columns past N read a valid row/column instead: they only
  // feed outputs that are never stored.  K-tail reads and the prefetch past
  // the last K step fall outside the descriptors' ranges and return 0.
  // A: thread (wave w, lane l) copies lane l of fragments w and w + 4:
  // row 16 f + l%16, k chunk l/16 of the step
  const rsrc_t a_rs = make_rsrc(A, (uint32_t)((size_t)a_rows * K * 2));
  const int a_kc = lane >> 4;
  uint32_t a_off[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int m = min(m0 + 16 * (wave + kGmWaves * s) + (lane & 15), M - 1);
    const uint32_t r = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
    a_off[s] = (r * (uint32_t)K + 8u * a_kc) * 2u;
  }
  // B: lane (g, c) of wave w reads rows k0 + 8g + r (r = 0..7) of the 16-byte
  // piece at columns cw .. cw + 7.  The K step moves the descriptor base (and
  // shrinks its range), so rows past K are outside it.
  const int g = lane >> 4;
  const int c = lane & 15;
  const int cw = n0 + wave * kGmWN + 8 * c;
  const bf16_t* We = W + (size_t)e * K * N;
  const uint32_t b_off = ((uint32_t)(8 * g) * N + (uint32_t)min(cw, N - 8)) * 2u;
  const uint32_t row_bytes = (uint32_t)N * 2u;

  auto gload_b = [&](int kt, u32x4_t (&rb)[8]) {
    const int k0 = min(kt * kGmBK, K);
    const rsrc_t rs = make_rsrc(We + (size_t)k0 * N, (uint32_t)(K - k0) * row_bytes);
#pragma unroll
    for (int r = 0; r < 8; ++r) rb[r] = buf_ld16(rs, b_off + (uint32_t)r * row_bytes);
  };
  auto gload_a = [&](int kt, u32x4_t (&ra)[2]) {
    const bool ok = kt * kGmBK + 8 * a_kc < K;
    const uint32_t kb = (uint32_t)kt * (kGmBK * 2);
#pragma unroll
    for (int s = 0; s < 2; ++s) ra[s] = buf_ld16(a_rs, ok ? a_off[s] + kb : kOutOfRange);
  };
  auto lstore = [&](int kt, const u32x4_t (&ra)[2]) {
    const int buf = kt % kGmLdsBufs;
    sm.a[buf][wave][lane] = ra[0];
    sm.a[buf][wave + kGmWaves][lane] = ra[1];
  };

  f32x4_t acc[8][8];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[mi][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Register rings (two sets each, used alternately, so the main loop is
  // unrolled twice and no ring needs a register copy: a copy of a register a
  // load is still writing would wait for every load): B of steps kt and kt+1
  // (the set of step kt is reloaded with step kt+2 once transposed) and A of
  // steps kt+2 and kt+3.  The A fragments F[mi] hold step kt and each is
  // reloaded with step kt+1 right after its last MFMA of step kt.
  u32x4_t Rb0[8], Rb1[8];
  u32x4_t Ra0[2], Ra1[2];
  u32x4_t F[8];

  // One K step kt: transpose B(kt); issue the loads of step kt+3 (A) and
  // kt+2 (B) -- A first: loads retire in order, so the store of A(kt+3) at
  // the next step then waits for A alone, and B keeps its two steps of
  // lead; multiply, reading the A fragments of kt+1 from LDS as those of
  // kt retire; store A(kt+2) into LDS; one barrier after the fifth of the
  // eight MFMA groups.
  // LDS ring: buffer (kt+1)%3 is read during step kt and buffer (kt+2)%3
  // written before step kt's barrier, which orders that write before the
  // reads of step kt+1.  Its previous reads (of step kt-2) all precede the
  // barrier of step kt-1, which precedes the write.
  // The scheduling fences keep each phase in order (a transpose hoisted next
  // to the loads it reads would wait on them) and interleave each fragment
  // read after the eight MFMAs that last use the register.
  auto step = [&](int kt, u32x4_t (&rb)[8], u32x4_t (&ra_load)[2], const u32x4_t (&ra_store)[2]) {
    u32x4_t bt[8];
    transpose8x8_b16(rb, bt);
    asm volatile("" ::"v"(bt[0]), "v"(bt[1]), "v"(bt[2]), "v"(bt[3]), "v"(bt[4]), "v"(bt[5]), "v"(bt[6]),
                 "v"(bt[7])
                 : "memory");
    __builtin_amdgcn_sched_barrier(0);
    gload_a(kt + 3, ra_load);
    gload_b(kt + 2, rb);
    const int nbuf = (kt + 1) % kGmLdsBufs;
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
    // The ten global loads are spread over the MFMAs before the barrier (a
    // burst of them would hold up the MFMA issue while the address unit
    // drains it); each LDS access before the barrier has a group of MFMAs
    // behind it, so the barrier's wait for them costs nothing.
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 global load
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 global load
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // 4 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);     // 2 LDS writes
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __syncthreads();
    F[4] = sm.a[nbuf][4][lane];
#pragma unroll
    for (int mi = 5; mi < 8; ++mi) {
      group(mi);
      F[mi] = sm.a[nbuf][mi][lane];
    }
  };

  // Prologue: the loads in the order the steps issue them (A(j+1) then
  // B(j)), so the wait counts of the first steps match the later ones.
  const int nk = (K + kGmBK - 1) / kGmBK;
  gload_a(0, Ra0);
  gload_a(1, Ra1);
  gload_b(0, Rb0);
  lstore(0, Ra0);
  gload_a(2, Ra0);
  gload_b(1, Rb1);
  lstore(1, Ra1);
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 8; ++mi) F[mi] = sm.a[0][mi][lane];

  // The step count is rounded up to the unroll period: an extra step reads
  // only zeros (K past the end of both descriptors) and adds exactly 0.
  const int nk2 = (nk + 1) / 2 * 2;
  for (int kt = 0; kt < nk2; kt += 2) {
    step(kt + 0, Rb0, Ra1, Ra0);
    step(kt + 1, Rb1, Ra0, Ra1);
  }

  // ---- epilogue.  16x16 accumulator layout: lane l, element v holds row
  // 4*(l/16) + v of MFMA column l%16 = weight column cw + j of operand j.
  // N % 8 == 0 and cw % 8 == 0: a lane's eight columns are all in range or
  // all out of it.
  if (cw >= N) return;                                       // no barrier follows
  float bb[8];
  {
    const uint32_t* bp = reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + cw);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t bw = bp[q];
      bb[2 * q] = bf16lo(bw);
      bb[2 * q + 1] = bf16hi(bw);
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
          for (int q = 0; q < 2; ++q) {
            const float h0 = clamped_glu(acc[mi][4 * q][v] + bb[4 * q], acc[mi][4 * q + 1][v] + bb[4 * q + 1]);
            const float h1 = clamped_glu(acc[mi][4 * q + 2][v] + bb[4 * q + 2], acc[mi][4 * q + 3][v] + bb[4 * q + 3]);
            hw[q] = pack_bf16x2(h0, h1);
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
hipError_t launch(const void* A, const void* W, const void* bias, const int32_t* cnt, const int32_t* off,
                  const int32_t* rows, int64_t T, int K, int N, int E, int k, void* out, hipStream_t stream) {
  const int64_t S = T * k;
  const int64_t a_rows = GATE_UP ? T : S;
  // 32-bit buffer offsets: the token operand and one expert's weight below
  // 2 GiB, so no in-range offset comes near kOutOfRange
  if (a_rows * K * 2 >= ((int64_t)1 << 31) || (int64_t)K * N * 2 >= ((int64_t)1 << 31))
    return hipErrorNotSupported;
  const int n_tiles = (N + kGmBN - 1) / kGmBN;
  const int64_t m_slots = (S + kGmBM - 1) / kGmBM + E;
  const int64_t blocks = (int64_t)n_tiles * m_slots;
  const int64_t grid = (blocks + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_expert_kernel<GATE_UP>), dim3((unsigned)grid), dim3(kGmThreads), 0, stream,
                     (const bf16_t*)A, (const bf16_t*)W, (const bf16_t*)bias, cnt, off, rows, K, N, E, k,
                     (int)a_rows, n_tiles, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gate_up(const void* x, const void* Wgu, const void* bgu, const int32_t* cnt,
                               const int32_t* off, const int32_t* rows, int64_t T, int H, int E, int k,
                               int I, void* h, hipStream_t stream) {
  return launch<true>(x, Wgu, bgu, cnt, off, rows, T, H, 2 * I, E, k, h, stream);
}

hipError_t launch_gemm_down(const void* h, const void* Wd, const void* bd, const int32_t* cnt,
                            const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                            hipStream_t stream) {
  return launch<false>(h, Wd, bd, cnt, off, nullptr, T, I, H, E, k, o, stream);
}

}  // namespace moe
