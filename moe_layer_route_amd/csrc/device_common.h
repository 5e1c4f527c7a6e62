// Device-side helpers shared by the gfx950 kernels of the MoE block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;                                         // bfloat16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));     // MFMA bf16 operand
typedef float f32x4_t __attribute__((ext_vector_type(4)));       // 16x16 MFMA accumulator
typedef float f32x16_t __attribute__((ext_vector_type(16)));     // 32x32 MFMA accumulator
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));    // 16-byte vector access
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
// low / high half of a packed pair of bf16
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16, round to nearest even (the gfx950 conversion
// instruction, v_cvt_pk_bf16_f32); NaN stays NaN (quiet).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// v_perm_b32 byte selection over {hi:a, lo:b}
__device__ __forceinline__ uint32_t perm_b32(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(a, b, sel);
}
// (lo16 of x) | (lo16 of y) << 16
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) { return perm_b32(y, x, 0x05040100u); }
// (hi16 of x) | (hi16 of y) << 16
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) { return perm_b32(y, x, 0x07060302u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// 8x8 transpose of 16-bit elements held as 8 rows of u32x4_t (8 bf16 each):
// out[j] holds column j of the input, element r in position r.
__device__ __forceinline__ void transpose8x8_b16(const u32x4_t (&in)[8], u32x4_t (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_t& r0 = in[2 * q];
      const u32x4_t& r1 = in[2 * q + 1];
      uint32_t a, b;
      switch (j >> 1) {
        case 0: a = r0.x; b = r1.x; break;
        case 1: a = r0.y; b = r1.y; break;
        case 2: a = r0.z; b = r1.z; break;
        default: a = r0.w; b = r1.w; break;
      }
      w[q] = (j & 1) ? pack_hi(a, b) : pack_lo(a, b);
    }
    out[j] = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// Clamped interleaved GLU of one (gate, up) pair, float32.  The clamps are
// compare-selects so that a NaN gate or up stays NaN (min/max instructions
// would return the bound).  The logistic uses the hardware exponential and
// reciprocal (about 1 ulp each; h is then rounded to bf16).
__device__ __forceinline__ float clamped_glu(float gate, float up) {
  const float g = gate > 7.0f ? 7.0f : gate;
  const float u = up > 7.0f ? 7.0f : (up < -7.0f ? -7.0f : up);
  const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-1.702f * g));
  return (u + 1.0f) * (g * s);
}

// Orders one wave's LDS accesses where its lanes exchange data through LDS:
// the accesses before it are done, as every lane of the wave sees them,
// before the accesses after it.  The LDS carries out one wave's operations
// in issue order, so this only keeps the compiler from moving a lane's
// accesses across it (whose addresses it could prove distinct); it adds no
// instruction.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// Tile order of the grouped expert GEMMs, one launch for all experts.  Expert e
// has ceil(cnt[e] / bm) M tiles x n_tiles N tiles.  Tiles go expert by expert;
// within an expert, blocks of at most mblock M tiles take each N tile in turn
// (the block's M tiles share that N tile's weight slab, and its N tiles share
// the block's token rows).  Block b runs on XCD b % 8, and consecutive tiles go
// to one XCD, whose L2 then serves both reuses.  Every lane of the calling wave
// gets the same expert, first row and N tile; false for a block past the last
// tile (the grid is an upper bound).  Experts 4 lane .. 4 lane + 3: E <= 256.
__device__ __forceinline__ bool grouped_gemm_tile(const int32_t* __restrict__ cnt, int E, int bm, int n_tiles,
                                                  int mblock, int lane, int& e, int& m0, int& nt) {
  constexpr int kXcdCount = 8;
  int mt[4], tc[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ee = lane * 4 + i;
    mt[i] = ee < E ? (cnt[ee] + bm - 1) / bm : 0;
    tc[i] = mt[i] * n_tiles;
    sum += tc[i];
  }
  const int incl = wave_incl_scan(sum, lane);
  const int R = __shfl(incl, kWave - 1, kWave);
  const int Q = (R + kXcdCount - 1) / kXcdCount;
  const int xi = (int)blockIdx.x / kXcdCount;
  const int L = (int)(blockIdx.x % kXcdCount) * Q + xi;
  int fe = -1, fm = 0, fn = 0;
  if (xi < Q && L < R) {
    int start = incl - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (L >= start && L < start + tc[i]) {
        const int t = L - start;
        const int mb = t / (mblock * n_tiles);
        const int rows_b = min(mblock, mt[i] - mb * mblock);
        const int t2 = t - mb * mblock * n_tiles;
        fe = lane * 4 + i;
        fm = (mb * mblock + t2 % rows_b) * bm;
        fn = t2 / rows_b;
      }
      start += tc[i];
    }
  }
  const uint64_t found = __ballot(fe >= 0);
  if (found == 0) return false;
  const int src = __ffsll((unsigned long long)found) - 1;
  e = __builtin_amdgcn_readfirstlane(__shfl(fe, src, kWave));
  m0 = __builtin_amdgcn_readfirstlane(__shfl(fm, src, kWave));
  nt = __builtin_amdgcn_readfirstlane(__shfl(fn, src, kWave));
  return true;
}

// Raw buffer descriptor words (base, byte range, stride 0) for the direct-to-LDS
// loads below; an offset at or past `bytes` reads 0 and touches no memory.
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// 16 bytes per lane from the buffer at voff + soff into LDS at lds + 16 * lane.
// Issued as assembly: the compiler would otherwise wait for every such load
// before any later LDS read.  M0 holds the LDS address (one wait state after
// writing it); the loads count in vmcnt and the waits are explicit.
__device__ __forceinline__ void dma16(u32x4_t rs, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(soff), "s"(lds)
               : "memory");
}
// The same with 4 bytes per lane, into LDS at lds + 4 * lane.
__device__ __forceinline__ void dma4(u32x4_t rs, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(soff), "s"(lds)
               : "memory");
}

// streaming (read-once) 16-byte load
__device__ __forceinline__ u32x4_t ldg16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

}  // namespace moe
