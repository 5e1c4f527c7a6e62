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
// ceil(T*k / BM) + E).  Each workgroup looks up which expert and which rows its
// M-tile slot holds from cnt[] (prefix sum of ceil(cnt[e] / BM)); surplus
// slots exit before any load or barrier.  Linear block ids are remapped so
// that consecutive tiles (the M tiles of one expert on one N tile, which share
// the weight slab) run on the same XCD, whose L2 serves the reuse.
//
// Tile: 128 rows x 512 columns, K steps of 32, eight waves (two per SIMD)
// side by side along N; each owns 128 rows x 64 columns = 8 x 4 tiles of
// v_mfma_f32_16x16x32_bf16 (128 fp32 accumulators per lane).
//   B (weight, [K][N] with N contiguous): no two waves share a column, so B
//     bypasses LDS.  Lane (g = lane/16, c = lane%16) of a wave loads rows
//     k0+8g .. k0+8g+7 of its 4 columns c0+4c .. c0+4c+3 (8-byte buffer loads,
//     two K steps ahead); an 8x4 transpose in registers turns them into four
//     K-packed B operands: operand j holds column c0+4c+j in MFMA column c.
//   A (token rows, k contiguous) is shared by the eight waves: gathered
//     through rows[] (gate_up) or contiguous rows of h (down), staged through
//     registers into two LDS buffers, one barrier per K step.  The buffers are
//     fragment-major: fragment mi (rows 16 mi .. 16 mi + 15) is 1 KB holding,
//     in lane order, the 16 bytes lane l of the MFMA needs (row l%16, k chunk
//     l/16), so every fragment read and every store is one contiguous 1 KB
//     access, free of bank conflicts.
// Epilogue: in the 16x16 accumulator layout lane l holds rows 4*(l/16)+0..3
// of MFMA column l%16, i.e. weight column c0+4c+j of operand j, so gate
// (j even) and up (j+1) of one pair sit in the same lane: bias + clamped GLU
// in registers, h stored as bf16 (gate_up); bias and float32 store (down).
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kGmThreads = 512;
constexpr int kGmBM = 128;
constexpr int kGmBN = 512;
constexpr int kGmBK = 32;
constexpr int kXcds = 8;


struct GemmSmem {
  u32x4_t a[2][kGmBM / 16][kWave];   // 2 x 8 fragments x 1 KB
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

struct Stage {
  u32x4_t a;
  u32x2_t b[8];
};

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ u32x2_t buf_ld8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}

template <bool GATE_UP>
__global__ __launch_bounds__(kGmThreads, 1) void gemm_expert_kernel(
    const bf16_t* __restrict__ A,      // gate_up: x [T][K]; down: h [S][K] (permuted order)
    const bf16_t* __restrict__ W,      // [E][K][N]
    const bf16_t* __restrict__ bias,   // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,  // gate_up: permuted slot ids
    int K, int N, int E, int kslots, int a_rows, int n_tiles, int m_slots, void* __restrict__ out) {
  __shared__ __align__(16) GemmSmem sm;
  __shared__ int s_tile[2];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

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
      tc[i] = e < E ? (cnt[e] + kGmBM - 1) / kGmBM : 0;
      sum += tc[i];
    }
    int start = wave_incl_scan(sum, lane) - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ms >= start && ms < start + tc[i]) {
        s_tile[0] = lane * 4 + i;
        s_tile[1] = (ms - start) * kGmBM;
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
  const int n0 = nt * kGmBN;

  // ---- per-thread global load assignments ----
  // Buffer loads: the descriptor (SGPRs) holds the base, each lane a constant
  // 32-bit offset, and the K step advances a uniform offset, which keeps the
  // VGPRs free for three stages of loads in flight.  Every load is
  // unconditional (a masked load becomes a branch, and the compiler then
  // drains all outstanding loads at the merge).  Rows past M and columns past
  // N read a valid row/column instead: they only feed outputs that are never
  // stored.  K-tail reads fall outside the descriptor's range and return 0.
  // A: thread t copies the 16 bytes lane t%64 of fragment t/64 holds: row
  // 16 (t/64) + t%16, k chunk (t/16)%4
  const rsrc_t a_rs = make_rsrc(A, (uint32_t)((size_t)a_rows * K * 2));
  const int a_row = 16 * wave + (lane & 15);
  const int a_kc = lane >> 4;
  uint32_t a_off;
  {
    const int m = min(m0 + a_row, M - 1);
    const uint32_t r = GATE_UP ? (uint32_t)(rows[row0 + m] / kslots) : (uint32_t)(row0 + m);
    a_off = (r * (uint32_t)K + 8u * a_kc) * 2u;
  }
  // B: lane (g, c) of wave w reads rows k0 + 8g + r (r = 0..7) of the 8-byte
  // piece at column n0 + 64 w + 4c
  const int g = lane >> 4;
  const int c = lane & 15;
  const rsrc_t b_rs = make_rsrc(W + (size_t)e * K * N, (uint32_t)((size_t)K * N * 2));
  const int b_gcol = n0 + wave * 64 + 4 * c;
  const uint32_t b_off = ((uint32_t)(8 * g) * N + (uint32_t)min(b_gcol, N - 4)) * 2u;

  auto gload = [&](int kt, Stage& st) {
    const int k0 = kt * kGmBK;
    const bool ok = k0 + 8 * a_kc < K;
    st.a = buf_ld16(a_rs, ok ? a_off + 2u * k0 : 0xFFFFFFF0u, 0);
    const uint32_t soff = (uint32_t)k0 * N * 2u;
#pragma unroll
    for (int r = 0; r < 8; ++r) st.b[r] = buf_ld8(b_rs, b_off + (uint32_t)r * N * 2u, soff);
  };
  auto lstore = [&](int buf, const Stage& st) { sm.a[buf][wave][lane] = st.a; };

  f32x4_t acc[8][4];
#pragma unroll
  for (int mi = 0; mi < 8; ++mi)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mi][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, const Stage& st) {
    // 8 x 4 transpose: operand j, dword q = (row 2q, row 2q+1) of column j
    u32x4_t bt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x0 = st.b[2 * q][j >> 1], x1 = st.b[2 * q + 1][j >> 1];
        w[q] = (j & 1) ? pack_hi(x0, x1) : pack_lo(x0, x1);
      }
      bt[j] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int mi = 0; mi < 8; ++mi) {
      const u32x4_t af = sm.a[buf][mi][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mi][j] = mfma16x16x32(af, bt[j], acc[mi][j]);
    }
  };

  const int nk = (K + kGmBK - 1) / kGmBK;
  Stage R0, R1, R2;
  gload(0, R0);
  gload(1, R1);
  lstore(0, R0);
  __syncthreads();
  // One K step: issue the loads two steps ahead, multiply the current step
  // (A from LDS, B from registers), move the next step's A into the other LDS
  // buffer.  Prefetch and store are unconditional: loads past K return 0 from
  // the buffer descriptors and land where nobody reads them, and a conditional
  // load would make the compiler wait for every outstanding load.
  // The scheduling fences keep the transpose of a stage inside its own step:
  // hoisted next to the loads it reads, it would force a wait on them.
  auto step = [&](int kt, const Stage& cur, const Stage& next, Stage& ahead) {
    gload(kt + 2, ahead);
    __builtin_amdgcn_sched_barrier(0);
    compute(kt & 1, cur);
    __builtin_amdgcn_sched_barrier(0);
    lstore((kt + 1) & 1, next);
    __syncthreads();
  };
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    step(kt, R0, R1, R2);
    step(kt + 1, R1, R2, R0);
    step(kt + 2, R2, R0, R1);
  }
  if (kt < nk) step(kt, R0, R1, R2);
  if (kt + 1 < nk) step(kt + 1, R1, R2, R0);

  // ---- epilogue.  16x16 accumulator layout: lane l, element v holds row
  // 4*(l/16) + v of MFMA column l%16 = weight column b_gcol + j of operand j.
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    const int n = b_gcol + j;
    const bool n_ok = n < N;
    float b0 = 0.f, b1 = 0.f;
    if (n_ok) {
      const uint32_t bw = *reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + n);
      b0 = bf16lo(bw);
      b1 = bf16hi(bw);
    }
#pragma unroll
    for (int mi = 0; mi < 8; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + mi * 16 + 4 * g + v;
        if (n_ok && m < M) {
          if (GATE_UP) {
            const float hv = clamped_glu(acc[mi][j][v] + b0, acc[mi][j + 1][v] + b1);
            reinterpret_cast<uint16_t*>(out)[(size_t)(row0 + m) * (N / 2) + n / 2] = (uint16_t)f32_to_bf16(hv);
          } else {
            *reinterpret_cast<float2*>(reinterpret_cast<float*>(out) + (size_t)(row0 + m) * N + n) =
                make_float2(acc[mi][j][v] + b0, acc[mi][j + 1][v] + b1);
          }
        }
      }
  }
}

template <bool GATE_UP>
hipError_t launch(const void* A, const void* W, const void* bias, const int32_t* cnt, const int32_t* off,
                  const int32_t* rows, int64_t T, int K, int N, int E, int k, void* out, hipStream_t stream) {
  const int64_t S = T * k;
  const int64_t a_rows = GATE_UP ? T : S;
  // 32-bit buffer offsets: one operand (or one expert's weight) below 4 GiB
  if (a_rows * K * 2 >= ((int64_t)1 << 32) || (int64_t)K * N * 2 >= ((int64_t)1 << 32))
    return hipErrorNotSupported;
  const int n_tiles = (N + kGmBN - 1) / kGmBN;
  const int64_t m_slots = (S + kGmBM - 1) / kGmBM + E;
  const int64_t blocks = (int64_t)n_tiles * m_slots;
  const int64_t grid = (blocks + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_expert_kernel<GATE_UP>), dim3((unsigned)grid), dim3(kGmThreads), 0, stream,
                     (const bf16_t*)A, (const bf16_t*)W, (const bf16_t*)bias, cnt, off, rows, K, N, E, k,
                     (int)a_rows, n_tiles, (int)m_slots, out);
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
