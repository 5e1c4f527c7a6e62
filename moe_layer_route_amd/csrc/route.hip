// Router of the gpt-oss MoE block: logits, top-k, softmax weights.
//
// xserv "Phase 19: gpt-oss-20b MoE support", section 1 ("MoE" row: the router
// is a plain Linear with bias) and section 2 (router -> top-k softmax, with the
// expert ids staying on the device).
//
// The decision rule: l[t][e] = sum_h x[t][h] Wr[e][h] + br[e] is rounded to
// float32 and the k largest are taken by (value desc, index asc).  The kernel
// reaches exactly that decision without computing every logit in float64:
//
//  1. One workgroup of 16 waves per 64 tokens (16 when E > 128).  Both operands are k-contiguous
//     (x rows and Wr rows), so they feed v_mfma_f32_16x16x32_bf16 straight from
//     memory: the A operand is 16 token rows, the B operand 16 router rows.
//     The waves split the work as (16-expert group) x (slice of K): with G
//     groups (G rounded up to a power of two), 16/G waves share a group and
//     each takes one K slice, so even a decode batch keeps 16 waves busy per
//     workgroup.  The slices are summed in LDS in a fixed order.  Next to the
//     logit each wave accumulates S[t][e] = sum_h |x[t][h]| |Wr[e][h]| with a
//     second MFMA on the operands with their sign bits cleared.
//  2. bf16 x bf16 products are exact in float32, so the only error of the MFMA
//     logit is its float32 accumulation; over 90 steps of 32 products it stays
//     below 128 u S (u = 2^-24), and adding the bias rounds once more.  Each
//     logit therefore carries a bound d[e] (twice that, plus two ulps).
//  3. Per token, a wave picks the top k by the float32 values and checks that
//     every expert outside is below the k-th by more than both bounds and that
//     consecutive picks are separated the same way.  Then the exact logits
//     round to float32 in the same order and the decision is the exact one.
//  4. Otherwise (near ties; a few tokens per thousand) the candidates whose
//     interval reaches the k-th are recomputed in float64 (exact products,
//     float64 sum), rounded to float32 and decided with the same key.
// Softmax weights over the k picks use the float64 logits when a token was
// recomputed, the float32 ones otherwise (their error is far below 1e-4).
// Small batches (T*E up to 64K logits) use a plain exact kernel instead, where
// latency, not arithmetic, sets the time.
#include "device_common.h"
#include "launch.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;
// Batches with at most this many logits take the exact float64 kernel (one
// workgroup per token); larger ones the MFMA kernel with exact refinement.
constexpr int64_t kExactRouteMaxLogits = 64 * 1024;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ u32x4_t abs_bf16x8(u32x4_t v) {
  const uint32_t m = 0x7FFF7FFFu;
  return u32x4_t{v[0] & m, v[1] & m, v[2] & m, v[3] & m};
}

// Monotone map of float32 to uint32 (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t make_key(float v, int e) {
  return ((uint64_t)order_key(v) << 32) | (uint64_t)(0xFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int key_expert(uint64_t k) { return (int)(0xFFFFu - (uint32_t)(k & 0xFFFFu)); }

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint64_t o = __shfl_xor(v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

// Exact-product, float64-sum logit of one (token, expert) pair by one wave.
// Each lane's chunks (8 columns, every 64th) are loaded ITERS at a time, all
// before the first product, so a row of up to 512 ITERS columns costs one
// memory round trip.
template <int ITERS>
__device__ double logit_f64(const bf16_t* __restrict__ xrow, const bf16_t* __restrict__ wrow, double bias,
                            int H, int lane) {
  const int nchunk = H / 8;
  double a0 = 0.0, a1 = 0.0;
  for (int c0 = 0; c0 < nchunk; c0 += kWave * ITERS) {
    u32x4_t xv[ITERS], wv[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int c = min(c0 + lane + kWave * it, nchunk - 1);   // clamped; the tail is left out below
      xv[it] = ld16(xrow + 8 * c);
      wv[it] = ld16(wrow + 8 * c);
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      if (c0 + lane + kWave * it < nchunk) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a0 = fma((double)bf16lo(xv[it][q]), (double)bf16lo(wv[it][q]), a0);
          a1 = fma((double)bf16hi(xv[it][q]), (double)bf16hi(wv[it][q]), a1);
        }
      }
    }
  }
  return wave_sum_f64(a0 + a1) + bias;
}

// TG = 16-token groups per workgroup (each B fragment feeds TG MFMAs).
template <int TG, int EMAX>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, const bf16_t* __restrict__ br, int T, int H,
    int E, int k, int groups_p2, int32_t* __restrict__ ids, float* __restrict__ wout) {
  constexpr int kRouteTok = 16 * TG;
  constexpr int kRouteDepth = TG == 1 ? 6 : 3;   // K steps of loads in flight (register budget)
  __shared__ float s_logit[kRouteTok][EMAX];
  __shared__ float s_abs[kRouteTok][EMAX];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int t0 = blockIdx.x * kRouteTok;
  const int g = lane >> 4;
  const int c = lane & 15;

  const int nk = (H + 31) / 32;
  const rsrc_t x_rs = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
  const rsrc_t w_rs = make_rsrc(Wr, (uint32_t)((size_t)E * H * 2));
  // float32 additions in sequence on the way to a logit (K steps of one
  // accumulator, the slice sums, the in-MFMA sums and the bias), never
  // counted below the 128 the error analysis was made for
  float err_steps;
  if constexpr (TG == 4) {
    // ---- phase 1, 64 tokens x up to 128 experts: each K step's x tile
    // (4 x 16 token rows) and router tile (8 x 16 expert rows) are loaded
    // once into fragment-major LDS (double buffered, inside s_logit) and wave
    // w multiplies token group w%4 with expert groups 2(w/4) and 2(w/4)+1 over
    // all of K.  Waves 0-11 each copy one 16-byte piece per K step (waves 0-3
    // x, 4-11 the router), two steps ahead.
    static_assert(EMAX == 128, "64-token router tile holds 128 experts");
    constexpr int kFr = 12;                                    // fragments per K step
    u32x4_t* stage = reinterpret_cast<u32x4_t*>(&s_logit[0][0]);   // [2][kFr][64], 24 KB
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const bool loader = wv < kFr;
    // waves 12-15 load wave 0's piece too and never store it: every load is
    // unconditional (a load under a branch makes the compiler wait for all
    // loads at the merge)
    const bool ld_x = wv < 4 || !loader;
    const rsrc_t ld_rs = ld_x ? x_rs : w_rs;
    const int ld_row = wv < 4 ? t0 + 16 * wv + c : loader ? 16 * (wv - 4) + c : t0 + c;
    const uint32_t ld_off = ((uint32_t)ld_row * H + 8u * g) * 2u;
    auto gload = [&](int kb, u32x4_t& r) {
      const bool k_ok = kb * 32 + 8 * g < H;
      r = buf_ld16(ld_rs, k_ok ? ld_off + 64u * kb : 0xFFFFFFF0u, 0);
    };
    auto lstore = [&](int buf, const u32x4_t& r) { stage[(buf * kFr + wv) * kWave + lane] = r; };
    const int ti = wave & 3, gp = wave >> 2;
    const bool act0 = 32 * gp < E, act1 = 32 * gp + 16 < E;   // wave-uniform
    f32x4_t acc2[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    f32x4_t aab2[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    auto compute = [&](int buf) {
      const u32x4_t* st = stage + buf * kFr * kWave + lane;
      const u32x4_t a = st[ti * kWave];
      const u32x4_t aa = abs_bf16x8(a);
      if (act0) {
        const u32x4_t b = st[(4 + 2 * gp) * kWave];
        acc2[0] = mfma16x16x32(a, b, acc2[0]);
        aab2[0] = mfma16x16x32(aa, abs_bf16x8(b), aab2[0]);
      }
      if (act1) {
        const u32x4_t b = st[(5 + 2 * gp) * kWave];
        acc2[1] = mfma16x16x32(a, b, acc2[1]);
        aab2[1] = mfma16x16x32(aa, abs_bf16x8(b), aab2[1]);
      }
    };
    // Step kb: load kb+2, multiply kb (buffer kb%2), store kb+1 (loaded one
    // step ago) into the other buffer, barrier.  The other buffer was last
    // read during step kb-1, before the previous barrier.  The step count is
    // rounded up to even: a step past the end reads zeros and adds 0.
    u32x4_t R0, R1;
    gload(0, R0);
    gload(1, R1);
    if (loader) lstore(0, R0);
    __syncthreads();
    const int nk2 = (nk + 1) / 2 * 2;
    for (int kb = 0; kb < nk2; kb += 2) {
      gload(kb + 2, R0);
      compute(0);
      if (loader) lstore(1, R1);
      __syncthreads();
      gload(kb + 3, R1);
      compute(1);
      if (loader) lstore(0, R0);
      __syncthreads();
    }
    // 16x16 accumulator layout: lane l, element v = token 16 ti + 4 (l/16) + v,
    // expert 16 (2 gp + q) + l%16.  The staging buffers are dead after the
    // last barrier above.
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = 16 * (2 * gp + q) + c;
      if (e < E)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tt = 16 * ti + 4 * g + v;
          s_logit[tt][e] = acc2[q][v];
          s_abs[tt][e] = aab2[q][v];
        }
    }
    __syncthreads();
    err_steps = fmaxf(128.f, (float)(nk2 + 40));
  } else {
    // ---- phase 1: this wave's 16 experts x 16 tokens over its slice of K
    const int grp = wave % groups_p2;              // 16-expert group
    const int ks = wave / groups_p2;               // K slice
    const int nslices = kRouteWaves / groups_p2;
    const int kb_begin = (nk * ks) / nslices;
    const int kb_end = (nk * (ks + 1)) / nslices;
    const uint32_t a_off = ((uint32_t)(t0 + c) * H + 8u * g) * 2u;   // + 16 H * 2 per token group
    const uint32_t b_off = ((uint32_t)(16 * grp + c) * H + 8u * g) * 2u;
    const bool active = 16 * grp < E;              // wave-uniform

    f32x4_t acc[TG], aab[TG];
#pragma unroll
    for (int i = 0; i < TG; ++i) {
      acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      aab[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (active) {
      // Loads run kRouteDepth steps ahead in a ring of registers.  All loads are
      // unconditional: rows past T or E read as 0 (outside the descriptors), and
      // K steps outside this wave's slice or past H are sent outside on purpose.
      // (The scalar offset operand must be wave-uniform, so the per-lane tests
      // go into the vector offset.)
      struct Ld { u32x4_t a[TG]; u32x4_t b; };
      Ld ring[kRouteDepth];
      auto load = [&](int kb, Ld& d) {
        const bool k_ok = kb < kb_end && kb * 32 + 8 * g < H;
        const uint32_t koff = 64u * kb;
#pragma unroll
        for (int i = 0; i < TG; ++i)
          d.a[i] = buf_ld16(x_rs, k_ok ? a_off + koff + (uint32_t)(32 * i) * H : 0xFFFFFFF0u, 0);
        d.b = buf_ld16(w_rs, k_ok ? b_off + koff : 0xFFFFFFF0u, 0);
      };
#pragma unroll
      for (int d = 0; d < kRouteDepth; ++d) load(kb_begin + d, ring[d]);
      for (int kb0 = kb_begin; kb0 < kb_end; kb0 += kRouteDepth) {
#pragma unroll
        for (int d = 0; d < kRouteDepth; ++d) {
          const u32x4_t bb = abs_bf16x8(ring[d].b);
#pragma unroll
          for (int i = 0; i < TG; ++i) {
            acc[i] = mfma16x16x32(ring[d].a[i], ring[d].b, acc[i]);
            aab[i] = mfma16x16x32(abs_bf16x8(ring[d].a[i]), bb, aab[i]);
          }
          load(kb0 + d + kRouteDepth, ring[d]);
        }
      }
    }
    // sum the K slices in slice order (16x16 accumulator layout: lane l,
    // element v = token 4*(l/16)+v, expert 16*grp + l%16)
    const int e_mine = 16 * grp + c;
    for (int s = 0; s < nslices; ++s) {
      if (s == ks && active && e_mine < E) {
#pragma unroll
        for (int i = 0; i < TG; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int tt = 16 * i + 4 * g + v;
            if (s == 0) {
              s_logit[tt][e_mine] = acc[i][v];
              s_abs[tt][e_mine] = aab[i][v];
            } else {
              s_logit[tt][e_mine] += acc[i][v];
              s_abs[tt][e_mine] += aab[i][v];
            }
          }
      }
      __syncthreads();
    }

    err_steps = fmaxf(128.f, (float)((nk + nslices - 1) / nslices + nslices + 40));
  }

  // ---- phase 2: one wave per token, waves take every 16th token ----
  constexpr int kPer = EMAX / kWave;             // experts per lane
  constexpr float u = 5.9604645e-8f;             // 2^-24
  float bias[kPer];                              // this lane's router biases, for every token
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + kWave * i;
    bias[i] = e < E ? bf16_to_f32(br[e]) : 0.f;
  }
  for (int tt = wave; tt < kRouteTok; tt += kRouteWaves) {
    const int t = t0 + tt;
    if (t >= T) break;                                       // wave-uniform, no barrier follows
    float lv[kPer], dv[kPer];
    uint64_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + kWave * i;
      key[i] = 0;
      lv[i] = -INFINITY;
      dv[i] = 0.f;
      if (e < E) {
        const float l = s_logit[tt][e] + bias[i];
        lv[i] = l;
        // error bound of the float32 logit, doubled, plus two ulps of it
        dv[i] = 2.f * (err_steps * u * s_abs[tt][e] + 2.f * u * fabsf(l)) + 2.4e-7f * fabsf(l) + 1e-30f;
        key[i] = make_key(l, e);
      }
    }
    // top k by the float32 values
    int sel[MOE_MAX_K_DEV];
    float sl[MOE_MAX_K_DEV], sd[MOE_MAX_K_DEV];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K_DEV; ++j) {
      sel[j] = 0;
      sl[j] = 0.f;
      sd[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_K_DEV; ++j) {
      if (j >= k) break;
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < kPer; ++i) best = key[i] > best ? key[i] : best;
      best = wave_max_u64(best);
      const int e = key_expert(best);
      sel[j] = e;
      float l = 0.f, d = 0.f;
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (lane + kWave * i == e) {
          key[i] = 0;
          l = lv[i];
          d = dv[i];
        }
      // broadcast from the owning lane
      sl[j] = __shfl(l, e % kWave, kWave);
      sd[j] = __shfl(d, e % kWave, kWave);
    }
    // certainty: every other expert strictly below the k-th interval, and the
    // picks pairwise separated
    const float cut = sl[k - 1] - sd[k - 1];
    float top_other = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (key[i] != 0) top_other = fmaxf(top_other, lv[i] + dv[i]);
    top_other = wave_max_f32(top_other);
    bool certain = top_other < cut;
#pragma unroll
    for (int j = 0; j + 1 < MOE_MAX_K_DEV; ++j)
      if (j + 1 < k) certain = certain && (sl[j] - sd[j] > sl[j + 1] + sd[j + 1]);

    double wl[MOE_MAX_K_DEV];
#pragma unroll
    for (int j = 0; j < MOE_MAX_K_DEV; ++j) wl[j] = 0.0;
    if (certain) {
#pragma unroll
      for (int j = 0; j < MOE_MAX_K_DEV; ++j) wl[j] = (double)sl[j];
    } else {
      // candidates: the picks and every expert whose interval reaches the cut
      const bf16_t* xrow = x + (size_t)t * H;
      double lx[kPer];
      uint64_t key2[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + kWave * i;
        bool cand = false;
        if (e < E) {
          bool picked = false;
#pragma unroll
          for (int j = 0; j < MOE_MAX_K_DEV; ++j) picked = picked || (j < k && sel[j] == e);
          cand = picked || (lv[i] + dv[i] >= cut);
        }
        uint64_t m = __ballot(cand);
        lx[i] = 0.0;
        key2[i] = 0;
        while (m) {                                          // wave-uniform loop
          const int src = __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          const int ec = src + kWave * i;
          // (fewer loads in flight for the 64-token variant: its registers are full)
          const double l64 =
              logit_f64<TG == 1 ? 8 : 4>(xrow, Wr + (size_t)ec * H, (double)bf16_to_f32(br[ec]), H, lane);
          if (lane == src) {
            lx[i] = l64;
            key2[i] = make_key((float)l64, ec);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < MOE_MAX_K_DEV; ++j) {
        if (j >= k) break;
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) best = key2[i] > best ? key2[i] : best;
        best = wave_max_u64(best);
        const int e = key_expert(best);
        sel[j] = e;
        double l = 0.0;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          if (lane + kWave * i == e) {
            key2[i] = 0;
            l = lx[i];
          }
        wl[j] = __shfl(l, e % kWave, kWave);
      }
    }
    // lane j < k takes pick j: one exponential per lane, summed across the
    // first k lanes in a fixed order (lane 0 + lane 1 + ...)
    int my = sel[0];
    double myl = wl[0];
#pragma unroll
    for (int j = 1; j < MOE_MAX_K_DEV; ++j)
      if (lane == j) {
        my = sel[j];
        myl = wl[j];
      }
    const double z = lane < k ? exp(myl - wl[0]) : 0.0;
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < MOE_MAX_K_DEV; ++j) sum += __shfl(z, j, kWave);
    if (lane < k) {
      ids[(size_t)t * k + lane] = my;
      wout[(size_t)t * k + lane] = (float)(z / sum);
    }
  }
}

// Small batches: one workgroup of 16 waves per token computes every logit
// exactly (exact products, float64 sum).  Wave w takes experts w, w+16, ...,
// two at a time; a unit of work is two experts x up to kExactIters chunks of
// 8 columns per lane.  Units alternate between two register sets: the loads
// of unit u+1 are in flight while unit u is multiplied, and the first unit is
// issued before the token's row of x lands in LDS.  Wave 0 then rounds the
// logits to float32, takes the top k by (value desc, index asc) and the
// softmax over the picks in float64.
constexpr int kExactBatch = 2;    // experts per unit
constexpr int kExactIters = 4;    // 16-byte chunks per lane and expert per unit

__global__ __launch_bounds__(kRouteThreads) void route_exact_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ Wr, const bf16_t* __restrict__ br, int H, int E,
    int k, int32_t* __restrict__ ids, float* __restrict__ wout) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* logit = reinterpret_cast<double*>(smem);                                  // [E]
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem + sizeof(double) * MOE_MAX_E_DEV);     // [H]
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nchunk = H / 8;
  const int ngrp = (nchunk + kWave * kExactIters - 1) / (kWave * kExactIters);   // chunk groups per expert
  const int nbatch = (E - wave + kRouteWaves * kExactBatch - 1) / (kRouteWaves * kExactBatch);
  const int units = nbatch * ngrp;   // wave-uniform; may be 0 when E < 16

  // unit u = (expert batch u / ngrp, chunk group u % ngrp).  Rows past E and
  // chunks past H read a valid row / chunk (clamped) that is never used.
  typedef u32x4_t Set[kExactBatch][kExactIters];
  auto load = [&](int u, Set& wv) {
    const int b = u / ngrp, g = u - (u / ngrp) * ngrp;
#pragma unroll
    for (int i = 0; i < kExactBatch; ++i) {
      const int e = min(wave + kRouteWaves * (kExactBatch * b + i), E - 1);
#pragma unroll
      for (int it = 0; it < kExactIters; ++it) {
        const int c = min(lane + kWave * (kExactIters * g + it), nchunk - 1);
        wv[i][it] = ld16(Wr + (size_t)e * H + 8 * c);
      }
    }
  };
  // two partial sums per expert (even and odd columns) for a shorter chain
  double acc[kExactBatch][2];
#pragma unroll
  for (int i = 0; i < kExactBatch; ++i) acc[i][0] = acc[i][1] = 0.0;
  auto compute = [&](int u, const Set& wv) {
    const int b = u / ngrp, g = u - (u / ngrp) * ngrp;
#pragma unroll
    for (int it = 0; it < kExactIters; ++it) {
      const int c = lane + kWave * (kExactIters * g + it);
      if (c < nchunk) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + 8 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const double xl = (double)bf16lo(xv[q]), xh = (double)bf16hi(xv[q]);
#pragma unroll
          for (int i = 0; i < kExactBatch; ++i) {
            acc[i][0] = fma(xl, (double)bf16lo(wv[i][it][q]), acc[i][0]);
            acc[i][1] = fma(xh, (double)bf16hi(wv[i][it][q]), acc[i][1]);
          }
        }
      }
    }
    if (g == ngrp - 1) {
#pragma unroll
      for (int i = 0; i < kExactBatch; ++i) {
        const double sum = wave_sum_f64(acc[i][0] + acc[i][1]);
        const int e = wave + kRouteWaves * (kExactBatch * b + i);
        if (lane == 0 && e < E) logit[e] = sum + (double)bf16_to_f32(br[e]);
        acc[i][0] = acc[i][1] = 0.0;
      }
    }
  };

  Set wa, wb;
  load(0, wa);
  const bf16_t* xrow = x + (size_t)t * H;
  for (int c = threadIdx.x; c < nchunk; c += kRouteThreads)
    *reinterpret_cast<u32x4_t*>(xs + 8 * c) = ld16(xrow + 8 * c);
  __syncthreads();
  for (int u = 0; u < units; u += 2) {
    load(u + 1, wb);   // past the last unit: clamped rows, never used
    compute(u, wa);
    load(u + 2, wa);
    if (u + 1 < units) compute(u + 1, wb);
  }
  __syncthreads();
  if (wave != 0) return;   // no barrier follows
  constexpr int kPer = MOE_MAX_E_DEV / kWave;
  uint64_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + kWave * i;
    key[i] = e < E ? make_key((float)logit[e], e) : 0;
  }
  int sel[MOE_MAX_K_DEV];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K_DEV; ++j) {
    sel[j] = 0;
    if (j >= k) break;
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = key_expert(best);
    sel[j] = e;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane + kWave * i == e) key[i] = 0;
  }
  // lane j < k takes pick j: one exponential per lane, summed across the
  // first k lanes in a fixed order (lane 0 + lane 1 + ...)
  int my = sel[0];
#pragma unroll
  for (int j = 1; j < MOE_MAX_K_DEV; ++j)
    if (lane == j) my = sel[j];
  const double z = lane < k ? exp(logit[my] - logit[sel[0]]) : 0.0;
  double sum = 0.0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_K_DEV; ++j) sum += __shfl(z, j, kWave);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my;
    wout[(size_t)t * k + lane] = (float)(z / sum);
  }
}

}  // namespace

hipError_t launch_route(const void* x, const void* Wr, const void* br, int64_t T, int H, int E, int k,
                        int32_t* ids, float* w, int method, hipStream_t stream) {
  if (method == 1 || (method == 0 && T * E <= kExactRouteMaxLogits)) {
    const size_t lds = sizeof(double) * MOE_MAX_E_DEV + sizeof(bf16_t) * (size_t)H;
    hipLaunchKernelGGL(route_exact_kernel, dim3((unsigned)T), dim3(kRouteThreads), lds, stream,
                       (const bf16_t*)x, (const bf16_t*)Wr, (const bf16_t*)br, H, E, k, ids, w);
    return hipGetLastError();
  }
  // 32-bit buffer offsets over x and Wr
  if (T * H * 2 >= ((int64_t)1 << 32) - 64) return hipErrorNotSupported;
  int groups_p2 = 1;
  while (groups_p2 * 16 < E) groups_p2 *= 2;   // E <= 256 -> at most 16 groups
  // 64 tokens per workgroup (each router fragment reused 4x) once there are
  // enough tokens to fill the chip that way and the LDS holds them (E <= 128)
  if (E <= 128 && T >= 8192) {
    const int64_t blocks = (T + 63) / 64;
    hipLaunchKernelGGL((route_kernel<4, 128>), dim3((unsigned)blocks), dim3(kRouteThreads), 0, stream,
                       (const bf16_t*)x, (const bf16_t*)Wr, (const bf16_t*)br, (int)T, H, E, k, groups_p2, ids, w);
  } else {
    const int64_t blocks = (T + 15) / 16;
    hipLaunchKernelGGL((route_kernel<1, MOE_MAX_E_DEV>), dim3((unsigned)blocks), dim3(kRouteThreads), 0, stream,
                       (const bf16_t*)x, (const bf16_t*)Wr, (const bf16_t*)br, (int)T, H, E, k, groups_p2, ids, w);
  }
  return hipGetLastError();
}

}  // namespace moe
