// Host-side launchers of the MoE block kernels (one per translation unit).
// They only enqueue; argument validation happens in the C ABI (moe_abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MOE_MAX_E_DEV 256
#define MOE_MAX_K_DEV 8

namespace moe {

// method: 0 = by size, 1 = exact float64 kernel, 2 = MFMA kernel with exact refinement
hipError_t launch_route(const void* x, const void* Wr, const void* br, int64_t T, int H, int E, int k,
                        int32_t* ids, float* w, int method, hipStream_t stream);

// e_begin: expert ids are counted from it; slots whose expert is outside
// [e_begin, e_begin + E) are skipped (pos = -1)
hipError_t launch_permute(const int32_t* ids, int64_t T, int E, int k, int32_t* cnt, int32_t* off,
                          int32_t* rows, int32_t* pos, hipStream_t stream, int e_begin = 0);
// slots of tokens t >= *n_valid (device int32) -> id -1, weight 0
hipError_t launch_mask_padding(int32_t* ids, float* w, int64_t T, int k, const int32_t* n_valid,
                               hipStream_t stream);

// Weight-streaming expert kernels (small token counts per expert).
hipError_t launch_gemv_gate_up(const void* x, const void* Wgu, const void* bgu, const int32_t* cnt,
                               const int32_t* off, const int32_t* rows, int64_t T, int H, int E, int k, int I,
                               void* h, hipStream_t stream);
hipError_t launch_gemv_down(const void* h, const void* Wd, const void* bd, const int32_t* cnt,
                            const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                            hipStream_t stream);

// LDS-tiled MFMA grouped GEMMs (large token counts per expert).
hipError_t launch_gemm_gate_up(const void* x, const void* Wgu, const void* bgu, const int32_t* cnt,
                               const int32_t* off, const int32_t* rows, int64_t T, int H, int E, int k,
                               int I, void* h, hipStream_t stream);
hipError_t launch_gemm_down(const void* h, const void* Wd, const void* bd, const int32_t* cnt,
                            const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                            hipStream_t stream);

// FP8 tiled GEMM staged through LDS by direct loads (fp8_gemm.hip); returns
// hipErrorNotSupported for K % 16 != 0 (or 2I % 64 != 0 for gate_up)
hipError_t launch_gemm_fp8_lds_gate_up(const void* xq, const float* sx, const void* Wq, const float* Ws,
                                       const void* bgu, const int32_t* cnt, const int32_t* off, const int32_t* rows,
                                       int64_t T, int H, int E, int k, int I, void* h, hipStream_t stream);
hipError_t launch_gemm_fp8_lds_down(const void* hq, const float* sh, const void* Wq, const float* Ws, const void* bd,
                                    const int32_t* cnt, const int32_t* off, int64_t T, int H, int E, int k, int I,
                                    float* o, hipStream_t stream);

// MXFP4 expert weights: codes [E][N][K/2], scales block-major [E][K/32][N] (K % 32 == 0)
hipError_t launch_mxfp4_quantize(const void* W, int E, int K, int N, void* codes, void* scales, hipStream_t stream);
hipError_t launch_mxfp4_gate_up(const void* x, const void* Wq, const void* Ws, const void* bgu, const int32_t* cnt,
                                const int32_t* off, const int32_t* rows, int64_t T, int H, int E, int k, int I,
                                void* h, hipStream_t stream);
hipError_t launch_mxfp4_down(const void* h, const void* Wq, const void* Ws, const void* bd, const int32_t* cnt,
                             const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                             hipStream_t stream);

hipError_t launch_gemm_mxfp4_gate_up(const void* x, const void* Wq, const void* Ws, const void* bgu,
                                     const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int H,
                                     int E, int k, int I, void* h, hipStream_t stream);
hipError_t launch_gemm_mxfp4_down(const void* h, const void* Wq, const void* Ws, const void* bd, const int32_t* cnt,
                                  const int32_t* off, int64_t T, int H, int E, int k, int I, float* o,
                                  hipStream_t stream);

// FP8 W8A8 (OCP E4M3): weight codes [E][N][K] with one float32 scale per
// expert; activation codes [R][K] with one scale per row (K % 16 == 0)
// R_live (device int32, optional): only rows below *R_live are quantised
hipError_t launch_fp8_quantize_rows(const void* a, int64_t R, int K, void* codes, float* scales, hipStream_t stream,
                                    const int32_t* R_live = nullptr);
hipError_t launch_fp8_quantize_weights(const void* W, int E, int K, int N, void* codes, float* scales,
                                       hipStream_t stream);
hipError_t launch_gemm_fp8_gate_up(const void* xq, const float* sx, const void* Wq, const float* Ws, const void* bgu,
                                   const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int H,
                                   int E, int k, int I, void* h, hipStream_t stream);
hipError_t launch_gemm_fp8_down(const void* hq, const float* sh, const void* Wq, const float* Ws, const void* bd,
                                const int32_t* cnt, const int32_t* off, int64_t T, int H, int E, int k, int I,
                                float* o, hipStream_t stream);
hipError_t launch_gemv_fp8_gate_up(const void* xq, const float* sx, const void* Wq, const float* Ws, const void* bgu,
                                   const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int H,
                                   int E, int k, int I, void* h, hipStream_t stream);
hipError_t launch_gemv_fp8_down(const void* hq, const float* sh, const void* Wq, const float* Ws, const void* bd,
                                const int32_t* cnt, const int32_t* off, int64_t T, int H, int E, int k, int I,
                                float* o, hipStream_t stream);

// measurement probes (probe.hip)
hipError_t launch_probe_mfma(int iters, int workgroups, float* out, hipStream_t stream);
hipError_t launch_probe_read(const void* buf, size_t bytes, int workgroups, uint32_t* out, hipStream_t stream);
hipError_t launch_probe_dot(const void* A, const void* B, int M, int K, float* out, hipStream_t stream);

// slots with pos < 0 are left out; out_f32: y is float32 (partial sums), else bf16
hipError_t launch_combine(const float* o, const int32_t* pos, const float* w, int64_t T, int H, int k,
                          void* y, hipStream_t stream, bool out_f32 = false);

}  // namespace moe
