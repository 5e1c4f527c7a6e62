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
// slots exit before any load.  Linear block ids are remapped so that
// consecutive tiles (the M tiles of one expert on one N tile, which share the
// weight slab) land on the same XCD, whose L2 then serves the reuse.
//
// Tile: BM x 256 output, K steps of 32, 4 waves in a 2 x 2 layout, each wave
// BM/2 x 128 with v_mfma_f32_32x32x16_bf16.  Both operands are staged in LDS
// as [row][k] with k contiguous (rows padded to 80 bytes, conflict-free
// 16-byte reads), double buffered with one barrier per K step:
//   A: token rows, gathered through rows[] (gate_up) or contiguous rows of h
//      (down), copied 16 bytes at a time;
//   B: the weight is stored [K][N] (N contiguous), so each thread loads a 4 x 8
//      block (4 k rows, 8 columns) and transposes it in registers into eight
//      4-element k runs, one per column.  For gate_up the columns are also
//      de-interleaved on the way into LDS: within every 64 columns, the 32
//      gate columns (even) come first and the 32 up columns (odd) second, so
//      MFMA tiles 2q and 2q+1 of a wave hold the gate and the up value of the
//      same (row, pair) in the same lane and the GLU epilogue is lane-local.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kGmThreads = 256;
constexpr int kGmBN = 256;
constexpr int kGmBK = 32;
constexpr int kGmLd = kGmBK + 8;   // LDS row pitch in bf16 (80 bytes)
constexpr int kXcds = 8;

template <int BM>
struct GemmSmem {
  bf16_t a[2][BM][kGmLd];
  bf16_t b[2][kGmBN][kGmLd];
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

template <int BM, bool GATE_UP>
__global__ __launch_bounds__(kGmThreads, 2) void gemm_expert_kernel(
    const bf16_t* __restrict__ A,      // gate_up: x [T][K]; down: h [S][K] (permuted order)
    const bf16_t* __restrict__ W,      // [E][K][N]
    const bf16_t* __restrict__ bias,   // [E][N]
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ off,
    const int32_t* __restrict__ rows,  // gate_up: permuted slot ids
    int K, int N, int E, int kslots, int n_tiles, int m_slots, void* __restrict__ out) {
  __shared__ __align__(16) GemmSmem<BM> sm;
  __shared__ int s_tile[2];

  constexpr int MI = BM / 64;          // 32-row MFMA tiles per wave along M
  constexpr int NI = 4;                // 32-column MFMA tiles per wave along N
  constexpr int A_CHUNKS = BM * (kGmBK / 8) / kGmThreads;   // 16-byte A chunks per thread

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
      tc[i] = e < E ? (cnt[e] + BM - 1) / BM : 0;
      sum += tc[i];
    }
    int start = wave_incl_scan(sum, lane) - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (ms >= start && ms < start + tc[i]) {
        s_tile[0] = lane * 4 + i;
        s_tile[1] = (ms - start) * BM;
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
  const bf16_t* a_ptr[A_CHUNKS];
  bool a_ok[A_CHUNKS];
  int a_row[A_CHUNKS], a_kc[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + kGmThreads * i;
    a_row[i] = c >> 2;
    a_kc[i] = c & 3;
    const int m = m0 + a_row[i];
    a_ok[i] = m < M;
    size_t r = 0;
    if (a_ok[i]) r = GATE_UP ? (size_t)(rows[row0 + m] / kslots) : (size_t)(row0 + m);
    a_ptr[i] = A + r * K + 8 * a_kc[i];
  }
  const int b_kq = tid >> 5;          // 4-row group of the K step (0..7)
  const int b_nb = tid & 31;          // 8-column group of the N tile (0..31)
  const bool b_ok = n0 + 8 * b_nb < N;
  const bf16_t* b_ptr = W + (size_t)e * K * N + (size_t)(4 * b_kq) * N + n0 + 8 * b_nb;
  int b_lrow[8];                      // LDS row of each of the thread's 8 columns
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pc = 8 * b_nb + j;
    b_lrow[j] = GATE_UP ? 64 * (pc >> 6) + 32 * (pc & 1) + ((pc & 63) >> 1) : pc;
  }

  const u32x4_t zero = {0u, 0u, 0u, 0u};
  u32x4_t ra[A_CHUNKS], rb[4];
  auto load_global = [&](int kt) {
    const int k0 = kt * kGmBK;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i)
      ra[i] = (a_ok[i] && k0 + 8 * a_kc[i] < K) ? ld16(a_ptr[i] + k0) : zero;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      rb[r] = (b_ok && k0 + 4 * b_kq + r < K) ? ldg16_stream(b_ptr + (size_t)(k0 + r) * N) : zero;
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i)
      *reinterpret_cast<u32x4_t*>(&sm.a[buf][a_row[i]][8 * a_kc[i]]) = ra[i];
    // 4 x 8 transpose: column j becomes the k run (r0[j], r1[j], r2[j], r3[j])
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int d = j >> 1;
      const uint32_t w0 = rb[0][d], w1 = rb[1][d], w2 = rb[2][d], w3 = rb[3][d];
      u32x2_t v;
      v[0] = (j & 1) ? pack_hi(w0, w1) : pack_lo(w0, w1);
      v[1] = (j & 1) ? pack_hi(w2, w3) : pack_lo(w2, w3);
      *reinterpret_cast<u32x2_t*>(&sm.b[buf][b_lrow[j]][4 * b_kq]) = v;
    }
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int frag_row = lane & 31;
  const int frag_k = 8 * (lane >> 5);
  const int nk = (K + kGmBK - 1) / kGmBK;

  load_global(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_global(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kGmBK / 16; ++ks) {
      u32x4_t af[MI], bfr[NI];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        af[mi] = *reinterpret_cast<const u32x4_t*>(
            &sm.a[buf][wm * (BM / 2) + mi * 32 + frag_row][ks * 16 + frag_k]);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        bfr[ni] = *reinterpret_cast<const u32x4_t*>(
            &sm.b[buf][wn * 128 + ni * 32 + frag_row][ks * 16 + frag_k]);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = mfma32x32x16(af[mi], bfr[ni], acc[mi][ni]);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  32x32 accumulator layout: lane l, element v holds
  // row 8*(v/4) + 4*(l/32) + v%4, column l%32 of the MFMA tile. ----
  const int col = lane & 31;
  const int rq = 4 * (lane >> 5);
  if (GATE_UP) {
    const int I = N / 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int i = n0 / 2 + wn * 64 + q * 32 + col;     // h column (gate/up pair)
      const bool i_ok = i < I;
      float bg = 0.f, bu = 0.f;
      if (i_ok) {
        const uint32_t bw = *reinterpret_cast<const uint32_t*>(bias + (size_t)e * N + 2 * i);
        bg = bf16lo(bw);
        bu = bf16hi(bw);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * (BM / 2) + mi * 32 + 8 * (v >> 2) + rq + (v & 3);
          if (i_ok && m < M) {
            const float hv = clamped_glu(acc[mi][2 * q][v] + bg, acc[mi][2 * q + 1][v] + bu);
            reinterpret_cast<uint16_t*>(out)[(size_t)(row0 + m) * I + i] = (uint16_t)f32_to_bf16(hv);
          }
        }
    }
  } else {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int n = n0 + wn * 128 + ni * 32 + col;
      const bool n_ok = n < N;
      const float bv = n_ok ? bf16_to_f32(bias[(size_t)e * N + n]) : 0.f;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * (BM / 2) + mi * 32 + 8 * (v >> 2) + rq + (v & 3);
          if (n_ok && m < M) reinterpret_cast<float*>(out)[(size_t)(row0 + m) * N + n] = acc[mi][ni][v] + bv;
        }
    }
  }
}

template <int BM, bool GATE_UP>
hipError_t launch(const void* A, const void* W, const void* bias, const int32_t* cnt, const int32_t* off,
                  const int32_t* rows, int64_t T, int K, int N, int E, int k, void* out, hipStream_t stream) {
  const int64_t S = T * k;
  const int n_tiles = (N + kGmBN - 1) / kGmBN;
  const int64_t m_slots = (S + BM - 1) / BM + E;
  const int64_t blocks = (int64_t)n_tiles * m_slots;
  const int64_t grid = (blocks + kXcds - 1) / kXcds * kXcds;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_expert_kernel<BM, GATE_UP>), dim3((unsigned)grid), dim3(kGmThreads), 0, stream,
                     (const bf16_t*)A, (const bf16_t*)W, (const bf16_t*)bias, cnt, off, rows, K, N, E, k,
                     n_tiles, (int)m_slots, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_gate_up(const void* x, const void* Wgu, const void* bgu, const int32_t* cnt,
                               const int32_t* off, const int32_t* rows, int64_t T, int H, int E, int k,
                               int I, void* h, hipStream_t stream) {
  return launch<128, true>(x, Wgu, bgu, cnt, off, rows, T, H, 2 * I, E, k, h, stream);
}

hipError_t launch_gemm_down(const void* h, const void* Wd, const void* bd, const int32_t* cnt,
                            const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                            hipStream_t stream) {
  return launch<128, false>(h, Wd, bd, cnt, off, nullptr, T, I, H, E, k, o, stream);
}

}  // namespace moe
