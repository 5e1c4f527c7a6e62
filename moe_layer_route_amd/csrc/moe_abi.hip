// C ABI of the MoE block: host-side argument checks, workspace layout and the
// per-call launch sequence.  Declared in include/moe_layer_route.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/moe_layer_route.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define CHECK_PTR(p, a)                                                                      \
  do {                                                                                       \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);          \
    if (!aligned((p), (a)))                                                                  \
      return fail(MOE_ERR_INVALID_ARG, "%s: %s is not %d-byte aligned", fn, #p, (int)(a));  \
  } while (0)

int check_dims(const char* fn, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T=%lld < 0", fn, (long long)T);
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, MOE_MAX_E);
  if (k < 1 || k > MOE_MAX_K || k > E)
    return fail(MOE_ERR_INVALID_ARG, "%s: k=%d outside [1, min(E=%d, %d)]", fn, k, E, MOE_MAX_K);
  if (H < 8 || H > MOE_MAX_DIM || H % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: H=%d must be a multiple of 8 in [8, %d]", fn, H, MOE_MAX_DIM);
  if (I < 8 || I > MOE_MAX_DIM || I % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: I=%d must be a multiple of 8 in [8, %d]", fn, I, MOE_MAX_DIM);
  if (T * (int64_t)k >= (int64_t)1 << 31)
    return fail(MOE_ERR_INVALID_ARG, "%s: T*k=%lld must be below 2^31", fn, (long long)(T * k));
  return MOE_OK;
}

int hip_status(const char* fn, hipError_t e) {
  if (e == hipErrorNotSupported) return fail(MOE_ERR_UNSUPPORTED, "%s: path not implemented", fn);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return MOE_OK;
}

struct Layout {
  size_t ids, w, cnt, off, rows, pos, h, o, total;
};

size_t take(size_t& cur, size_t bytes) {
  const size_t at = cur;
  cur += (bytes + 255) & ~(size_t)255;
  return at;
}

Layout layout(int64_t T, int32_t H, int32_t E, int32_t k, int32_t I) {
  Layout L;
  size_t cur = 0;
  const size_t S = (size_t)T * k;
  L.ids = take(cur, S * 4);
  L.w = take(cur, S * 4);
  L.cnt = take(cur, (size_t)E * 4);
  L.off = take(cur, (size_t)(E + 1) * 4);
  L.rows = take(cur, S * 4);
  L.pos = take(cur, S * 4);
  L.h = take(cur, S * I * 2);
  L.o = take(cur, S * H * 4);
  L.total = cur;
  return L;
}

// Mean rows per expert above which the tiled MFMA path is used.
constexpr int64_t kGemmMinMeanRows = 48;

// Expert path from host-known sizes only (no device read-back): the weight
// streaming path while each expert sees few rows, the tiled MFMA path once the
// mean load per expert makes the GEMMs compute-bound.
int choose_path(int32_t path, int64_t T, int32_t E, int32_t k) {
  if (path != MOE_PATH_AUTO) return path;
  return T * k > kGemmMinMeanRows * E ? MOE_PATH_GEMM : MOE_PATH_GEMV;
}

int run_gate_up(const char* fn, const void* x, const void* Wgu, const void* bgu, const int32_t* cnt,
                const int32_t* off, const int32_t* rows, int64_t T, int32_t H, int32_t E, int32_t k,
                int32_t I, void* h, int32_t path, hipStream_t s) {
  path = choose_path(path, T, E, k);
  if (path == MOE_PATH_GEMV)
    return hip_status(fn, moe::launch_gemv_gate_up(x, Wgu, bgu, cnt, off, rows, T, H, E, k, I, h, s));
  if (path == MOE_PATH_GEMM)
    return hip_status(fn, moe::launch_gemm_gate_up(x, Wgu, bgu, cnt, off, rows, T, H, E, k, I, h, s));
  return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
}

int run_down(const char* fn, const void* h, const void* Wd, const void* bd, const int32_t* cnt,
             const int32_t* off, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, float* o,
             int32_t path, hipStream_t s) {
  path = choose_path(path, T, E, k);
  if (path == MOE_PATH_GEMV)
    return hip_status(fn, moe::launch_gemv_down(h, Wd, bd, cnt, off, T, H, E, k, I, o, s));
  if (path == MOE_PATH_GEMM)
    return hip_status(fn, moe::launch_gemm_down(h, Wd, bd, cnt, off, T, H, E, k, I, o, s));
  return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
}


// ---------------------------------------------------------------------------
// Scratch of the allocation-free forward: a file-scope device array (each GPU
// the library runs on holds its own copy until the process ends).  In host
// code its name is only a stand-in for the symbol, so the device address is
// looked up once per device with that device current and kept; kernels and
// every host call get that address, never the name.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

int scratch_on_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device %d is beyond the %d the library tracks", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Host-side checks of the whole forward's arguments (nothing is enqueued).
int check_forward(const char* fn, const void* x, const void* Wr, const void* br, const void* Wgu, const void* bgu,
                  const void* Wd, const void* bd, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                  const void* y, const int32_t* topk_ids_out, const float* topk_w_out, int32_t path) {
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  CHECK_PTR(x, 16);
  CHECK_PTR(Wr, 16);
  CHECK_PTR(br, 2);
  CHECK_PTR(Wgu, 16);
  CHECK_PTR(bgu, 4);
  CHECK_PTR(Wd, 16);
  CHECK_PTR(bd, 4);
  CHECK_PTR(y, 16);
  if (topk_ids_out && !aligned(topk_ids_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_ids_out is not 4-byte aligned", fn);
  if (topk_w_out && !aligned(topk_w_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_w_out is not 4-byte aligned", fn);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  return MOE_OK;
}

// The whole forward on a caller-provided (or the library's own) workspace.
int forward_impl(const char* fn, const void* x, const void* Wr, const void* br, const void* Wgu, const void* bgu,
                 const void* Wd, const void* bd, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, void* y,
                 int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes, int32_t path,
                 void* stream) {
  if (int st = check_forward(fn, x, Wr, br, Wgu, bgu, Wd, bd, T, H, E, k, I, y, topk_ids_out, topk_w_out, path))
    return st;
  if (T == 0) return ok();
  const Layout L = layout(T, H, E, k, I);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, L.total);
  if (!aligned(workspace, 256))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.cnt);
  int32_t* off = reinterpret_cast<int32_t*>(ws + L.off);
  int32_t* rows = reinterpret_cast<int32_t*>(ws + L.rows);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  void* h = ws + L.h;
  float* o = reinterpret_cast<float*>(ws + L.o);
  hipStream_t s = (hipStream_t)stream;

  if (int st = hip_status(fn, moe::launch_route(x, Wr, br, T, H, E, k, ids, w, MOE_ROUTE_AUTO, s))) return st;
  if (int st = hip_status(fn, moe::launch_permute(ids, T, E, k, cnt, off, rows, pos, s))) return st;
  if (int st = run_gate_up(fn, x, Wgu, bgu, cnt, off, rows, T, H, E, k, I, h, path, s)) return st;
  if (int st = run_down(fn, h, Wd, bd, cnt, off, T, H, E, k, I, o, path, s)) return st;
  if (int st = hip_status(fn, moe::launch_combine(o, pos, w, T, H, k, y, s))) return st;
  return ok();
}


}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

int moe_expert_path(int64_t T, int32_t E, int32_t k) { return choose_path(MOE_PATH_AUTO, T, E, k); }

size_t moe_workspace_bytes(int64_t T, int32_t H, int32_t E, int32_t k, int32_t I) {
  if (check_dims("moe_workspace_bytes", T, H, E, k, I) != MOE_OK) return 0;
  if (T == 0) return 0;
  return layout(T, H, E, k, I).total;
}

int moe_route_ex(const void* x, const void* Wr, const void* br, int64_t T, int32_t H, int32_t E, int32_t k,
                 int32_t* topk_ids, float* topk_w, int32_t method, void* stream) {
  const char* fn = "moe_route";
  // I only has to be valid for the shared check; the router does not use it.
  if (int st = check_dims(fn, T, H, E, k, 8)) return st;
  CHECK_PTR(x, 16);
  CHECK_PTR(Wr, 16);
  CHECK_PTR(br, 2);
  CHECK_PTR(topk_ids, 4);
  CHECK_PTR(topk_w, 4);
  if (method < MOE_ROUTE_AUTO || method > MOE_ROUTE_MFMA)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown router method %d", fn, method);
  if (T == 0) return ok();
  if (int st = hip_status(fn, moe::launch_route(x, Wr, br, T, H, E, k, topk_ids, topk_w, method,
                                                (hipStream_t)stream)))
    return st;
  return ok();
}

int moe_route(const void* x, const void* Wr, const void* br, int64_t T, int32_t H, int32_t E, int32_t k,
              int32_t* topk_ids, float* topk_w, void* stream) {
  return moe_route_ex(x, Wr, br, T, H, E, k, topk_ids, topk_w, MOE_ROUTE_AUTO, stream);
}

int moe_forward_ex(const void* x, const void* Wr, const void* br, const void* Wgu, const void* bgu,
                   const void* Wd, const void* bd, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                   void* y, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                   size_t workspace_bytes, int32_t path, void* stream) {
  return forward_impl("moe_forward", x, Wr, br, Wgu, bgu, Wd, bd, T, H, E, k, I, y, topk_ids_out, topk_w_out,
                      workspace, workspace_bytes, path, stream);
}

int moe_forward_noalloc(const void* x, const void* Wr, const void* br, const void* Wgu, const void* bgu,
                        const void* Wd, const void* bd, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                        void* y, int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  const char* fn = "moe_forward_noalloc";
  if (int st = check_forward(fn, x, Wr, br, Wgu, bgu, Wd, bd, T, H, E, k, I, y, topk_ids_out, topk_w_out,
                             MOE_PATH_AUTO))
    return st;
  if (T == 0) return ok();
  const size_t need = layout(T, H, E, k, I).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_INVALID_ARG,
                "%s: T=%lld, H=%d, E=%d, k=%d, I=%d need %zu bytes of scratch; the library's array holds %zu "
                "(about T*k*(2I + 4H + 16) bytes are needed): use moe_forward with a workspace",
                fn, (long long)T, H, E, k, I, need, kScratchBytes);
  void* ws = nullptr;
  if (int st = scratch_on_current_device(fn, &ws)) return st;
  return forward_impl(fn, x, Wr, br, Wgu, bgu, Wd, bd, T, H, E, k, I, y, topk_ids_out, topk_w_out, ws,
                      kScratchBytes, MOE_PATH_AUTO, stream);
}

int moe_forward_ep(const void* x, const void* Wr, const void* br, const void* Wgu_local, const void* bgu_local,
                   const void* Wd_local, const void* bd_local, int64_t T, int32_t H, int32_t E, int32_t k,
                   int32_t I, int32_t e_begin, int32_t n_local, float* y_partial, int32_t* topk_ids_out,
                   float* topk_w_out, void* workspace, size_t workspace_bytes, int32_t path, void* stream) {
  const char* fn = "moe_forward_ep";
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  if (n_local < 1 || e_begin < 0 || e_begin > E - n_local)
    return fail(MOE_ERR_INVALID_ARG, "%s: local experts [%d, %d + %d) outside [0, E=%d)", fn, e_begin, e_begin,
                n_local, E);
  CHECK_PTR(x, 16);
  CHECK_PTR(Wr, 16);
  CHECK_PTR(br, 2);
  CHECK_PTR(Wgu_local, 16);
  CHECK_PTR(bgu_local, 4);
  CHECK_PTR(Wd_local, 16);
  CHECK_PTR(bd_local, 4);
  CHECK_PTR(y_partial, 16);
  if (topk_ids_out && !aligned(topk_ids_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_ids_out is not 4-byte aligned", fn);
  if (topk_w_out && !aligned(topk_w_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_w_out is not 4-byte aligned", fn);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  const Layout L = layout(T, H, E, k, I);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, L.total);
  if (!aligned(workspace, 256))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + L.cnt);
  int32_t* off = reinterpret_cast<int32_t*>(ws + L.off);
  int32_t* rows = reinterpret_cast<int32_t*>(ws + L.rows);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  void* h = ws + L.h;
  float* o = reinterpret_cast<float*>(ws + L.o);
  hipStream_t s = (hipStream_t)stream;
  // the expert path follows the whole layer's load per expert, T*k/E
  path = choose_path(path, T, E, k);

  if (int st = hip_status(fn, moe::launch_route(x, Wr, br, T, H, E, k, ids, w, MOE_ROUTE_AUTO, s))) return st;
  if (int st = hip_status(fn, moe::launch_permute(ids, T, n_local, k, cnt, off, rows, pos, s, e_begin))) return st;
  if (int st = run_gate_up(fn, x, Wgu_local, bgu_local, cnt, off, rows, T, H, n_local, k, I, h, path, s)) return st;
  if (int st = run_down(fn, h, Wd_local, bd_local, cnt, off, T, H, n_local, k, I, o, path, s)) return st;
  if (int st = hip_status(fn, moe::launch_combine(o, pos, w, T, H, k, y_partial, s, true))) return st;
  return ok();
}

int moe_forward_padded(const void* x, const void* Wr, const void* br, const void* Wgu, const void* bgu,
                       const void* Wd, const void* bd, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                       const int32_t* n_valid, void* y, int32_t* topk_ids_out, float* topk_w_out,
                       int32_t* expert_counts_out, void* workspace, size_t workspace_bytes, int32_t path,
                       void* stream) {
  const char* fn = "moe_forward_padded";
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  CHECK_PTR(x, 16);
  CHECK_PTR(Wr, 16);
  CHECK_PTR(br, 2);
  CHECK_PTR(Wgu, 16);
  CHECK_PTR(bgu, 4);
  CHECK_PTR(Wd, 16);
  CHECK_PTR(bd, 4);
  CHECK_PTR(y, 16);
  if (n_valid && !aligned(n_valid, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: n_valid is not 4-byte aligned", fn);
  if (topk_ids_out && !aligned(topk_ids_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_ids_out is not 4-byte aligned", fn);
  if (topk_w_out && !aligned(topk_w_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_w_out is not 4-byte aligned", fn);
  if (expert_counts_out && !aligned(expert_counts_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: expert_counts_out is not 4-byte aligned", fn);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  const Layout L = layout(T, H, E, k, I);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, L.total);
  if (!aligned(workspace, 256))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* cnt = expert_counts_out ? expert_counts_out : reinterpret_cast<int32_t*>(ws + L.cnt);
  int32_t* off = reinterpret_cast<int32_t*>(ws + L.off);
  int32_t* rows = reinterpret_cast<int32_t*>(ws + L.rows);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  void* h = ws + L.h;
  float* o = reinterpret_cast<float*>(ws + L.o);
  hipStream_t s = (hipStream_t)stream;

  if (int st = hip_status(fn, moe::launch_route(x, Wr, br, T, H, E, k, ids, w, MOE_ROUTE_AUTO, s))) return st;
  if (n_valid)
    if (int st = hip_status(fn, moe::launch_mask_padding(ids, w, T, k, n_valid, s))) return st;
  if (int st = hip_status(fn, moe::launch_permute(ids, T, E, k, cnt, off, rows, pos, s))) return st;
  if (int st = run_gate_up(fn, x, Wgu, bgu, cnt, off, rows, T, H, E, k, I, h, path, s)) return st;
  if (int st = run_down(fn, h, Wd, bd, cnt, off, T, H, E, k, I, o, path, s)) return st;
  if (int st = hip_status(fn, moe::launch_combine(o, pos, w, T, H, k, y, s))) return st;
  return ok();
}

int moe_forward(const void* x, const void* Wr, const void* br, const void* Wgu, const void* bgu,
                const void* Wd, const void* bd, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                void* y, int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                void* stream) {
  return moe_forward_ex(x, Wr, br, Wgu, bgu, Wd, bd, T, H, E, k, I, y, topk_ids_out, topk_w_out, workspace,
                        workspace_bytes, MOE_PATH_AUTO, stream);
}

int moe_permute(const int32_t* topk_ids, int64_t T, int32_t E, int32_t k, int32_t* cnt, int32_t* off,
                int32_t* rows, int32_t* pos, void* stream) {
  const char* fn = "moe_permute";
  if (int st = check_dims(fn, T, 8, E, k, 8)) return st;
  CHECK_PTR(topk_ids, 4);
  CHECK_PTR(cnt, 4);
  CHECK_PTR(off, 4);
  CHECK_PTR(rows, 4);
  CHECK_PTR(pos, 4);
  if (T == 0) return ok();
  if (int st = hip_status(fn, moe::launch_permute(topk_ids, T, E, k, cnt, off, rows, pos,
                                                  (hipStream_t)stream)))
    return st;
  return ok();
}

int moe_gate_up(const void* x, const void* Wgu, const void* bgu, const int32_t* cnt, const int32_t* off,
                const int32_t* rows, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, void* h,
                int32_t path, void* stream) {
  const char* fn = "moe_gate_up";
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  CHECK_PTR(x, 16);
  CHECK_PTR(Wgu, 16);
  CHECK_PTR(bgu, 4);
  CHECK_PTR(cnt, 4);
  CHECK_PTR(off, 4);
  CHECK_PTR(rows, 4);
  CHECK_PTR(h, 16);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  if (int st = run_gate_up(fn, x, Wgu, bgu, cnt, off, rows, T, H, E, k, I, h, path, (hipStream_t)stream))
    return st;
  return ok();
}

int moe_down(const void* h, const void* Wd, const void* bd, const int32_t* cnt, const int32_t* off,
             int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, float* o, int32_t path, void* stream) {
  const char* fn = "moe_down";
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  CHECK_PTR(h, 16);
  CHECK_PTR(Wd, 16);
  CHECK_PTR(bd, 4);
  CHECK_PTR(cnt, 4);
  CHECK_PTR(off, 4);
  CHECK_PTR(o, 16);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  if (int st = run_down(fn, h, Wd, bd, cnt, off, T, H, E, k, I, o, path, (hipStream_t)stream)) return st;
  return ok();
}

// ---------------------------------------------------------------------------
// MXFP4 expert weights
// ---------------------------------------------------------------------------
static int check_mx_dims(const char* fn, int32_t H, int32_t I) {
  if (H % 32 != 0 || I % 32 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: H=%d and I=%d must be multiples of 32 (MXFP4 blocks)", fn, H, I);
  return MOE_OK;
}

int moe_quantize_mxfp4(const void* W, int32_t E, int32_t K, int32_t N, void* codes, void* scales, void* stream) {
  const char* fn = "moe_quantize_mxfp4";
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, MOE_MAX_E);
  if (K < 32 || K > MOE_MAX_DIM || K % 32 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 32 in [32, %d]", fn, K, MOE_MAX_DIM);
  if (N < 8 || N > 2 * MOE_MAX_DIM || N % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: N=%d must be a multiple of 8 in [8, %d]", fn, N, 2 * MOE_MAX_DIM);
  CHECK_PTR(W, 2);
  CHECK_PTR(codes, 16);
  CHECK_PTR(scales, 1);
  if (int st = hip_status(fn, moe::launch_mxfp4_quantize(W, E, K, N, codes, scales, (hipStream_t)stream))) return st;
  return ok();
}

static int run_gate_up_mx(const char* fn, const void* x, const void* Wq, const void* Ws, const void* bgu,
                          const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int32_t H, int32_t E,
                          int32_t k, int32_t I, void* h, int32_t path, hipStream_t s) {
  path = choose_path(path, T, E, k);
  if (path == MOE_PATH_GEMV)
    return hip_status(fn, moe::launch_mxfp4_gate_up(x, Wq, Ws, bgu, cnt, off, rows, T, H, E, k, I, h, s));
  if (path == MOE_PATH_GEMM)
    return hip_status(fn, moe::launch_gemm_mxfp4_gate_up(x, Wq, Ws, bgu, cnt, off, rows, T, H, E, k, I, h, s));
  return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
}

static int run_down_mx(const char* fn, const void* h, const void* Wq, const void* Ws, const void* bd,
                       const int32_t* cnt, const int32_t* off, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                       float* o, int32_t path, hipStream_t s) {
  path = choose_path(path, T, E, k);
  if (path == MOE_PATH_GEMV)
    return hip_status(fn, moe::launch_mxfp4_down(h, Wq, Ws, bd, cnt, off, T, H, E, k, I, o, s));
  if (path == MOE_PATH_GEMM)
    return hip_status(fn, moe::launch_gemm_mxfp4_down(h, Wq, Ws, bd, cnt, off, T, H, E, k, I, o, s));
  return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
}

// The MXFP4 forward; n_valid (device, optional) marks the rows from *n_valid
// on as padding, expert_counts_out (optional) receives the per-expert loads.
static int forward_mxfp4(const char* fn, const void* x, const void* Wr, const void* br, const void* Wgu_q,
                         const void* Wgu_s, const void* bgu, const void* Wd_q, const void* Wd_s, const void* bd,
                         int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, int32_t e_begin, int32_t n_local,
                         const int32_t* n_valid, void* y, bool partial,
                         int32_t* topk_ids_out, float* topk_w_out, int32_t* expert_counts_out, void* workspace,
                         size_t workspace_bytes, int32_t path, void* stream) {
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  if (n_local < 1 || e_begin < 0 || e_begin > E - n_local)
    return fail(MOE_ERR_INVALID_ARG, "%s: local experts [%d, %d + %d) outside [0, E=%d)", fn, e_begin, e_begin,
                n_local, E);
  if (int st = check_mx_dims(fn, H, I)) return st;
  CHECK_PTR(x, 16);
  CHECK_PTR(Wr, 16);
  CHECK_PTR(br, 2);
  CHECK_PTR(Wgu_q, 16);
  CHECK_PTR(Wgu_s, 16);
  CHECK_PTR(bgu, 4);
  CHECK_PTR(Wd_q, 16);
  CHECK_PTR(Wd_s, 16);
  CHECK_PTR(bd, 4);
  CHECK_PTR(y, 16);
  if (topk_ids_out && !aligned(topk_ids_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_ids_out is not 4-byte aligned", fn);
  if (topk_w_out && !aligned(topk_w_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_w_out is not 4-byte aligned", fn);
  if (n_valid && !aligned(n_valid, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: n_valid is not 4-byte aligned", fn);
  if (expert_counts_out && !aligned(expert_counts_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: expert_counts_out is not 4-byte aligned", fn);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  const Layout L = layout(T, H, E, k, I);
  if (workspace == nullptr || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, L.total);
  if (!aligned(workspace, 256))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  char* ws = static_cast<char*>(workspace);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* cnt = expert_counts_out ? expert_counts_out : reinterpret_cast<int32_t*>(ws + L.cnt);
  int32_t* off = reinterpret_cast<int32_t*>(ws + L.off);
  int32_t* rows = reinterpret_cast<int32_t*>(ws + L.rows);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  void* h = ws + L.h;
  float* o = reinterpret_cast<float*>(ws + L.o);
  hipStream_t s = (hipStream_t)stream;
  // the expert path follows the whole layer's load per expert, T*k/E
  path = choose_path(path, T, E, k);

  if (int st = hip_status(fn, moe::launch_route(x, Wr, br, T, H, E, k, ids, w, MOE_ROUTE_AUTO, s))) return st;
  if (n_valid)
    if (int st = hip_status(fn, moe::launch_mask_padding(ids, w, T, k, n_valid, s))) return st;
  if (int st = hip_status(fn, moe::launch_permute(ids, T, n_local, k, cnt, off, rows, pos, s, e_begin))) return st;
  if (int st = run_gate_up_mx(fn, x, Wgu_q, Wgu_s, bgu, cnt, off, rows, T, H, n_local, k, I, h, path, s)) return st;
  if (int st = run_down_mx(fn, h, Wd_q, Wd_s, bd, cnt, off, T, H, n_local, k, I, o, path, s)) return st;
  if (int st = hip_status(fn, moe::launch_combine(o, pos, w, T, H, k, y, s, partial))) return st;
  return ok();
}

int moe_forward_mxfp4_ex(const void* x, const void* Wr, const void* br, const void* Wgu_q, const void* Wgu_s,
                         const void* bgu, const void* Wd_q, const void* Wd_s, const void* bd, int64_t T, int32_t H,
                         int32_t E, int32_t k, int32_t I, void* y, int32_t* topk_ids_out, float* topk_w_out,
                         void* workspace, size_t workspace_bytes, int32_t path, void* stream) {
  return forward_mxfp4("moe_forward_mxfp4", x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, T, H, E, k, I, 0, E,
                       nullptr, y, false, topk_ids_out, topk_w_out, nullptr, workspace, workspace_bytes, path, stream);
}

int moe_forward_padded_mxfp4(const void* x, const void* Wr, const void* br, const void* Wgu_q, const void* Wgu_s,
                             const void* bgu, const void* Wd_q, const void* Wd_s, const void* bd, int64_t T,
                             int32_t H, int32_t E, int32_t k, int32_t I, const int32_t* n_valid, void* y,
                             int32_t* topk_ids_out, float* topk_w_out, int32_t* expert_counts_out, void* workspace,
                             size_t workspace_bytes, int32_t path, void* stream) {
  return forward_mxfp4("moe_forward_padded_mxfp4", x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, T, H, E, k, I,
                       0, E, n_valid, y, false, topk_ids_out, topk_w_out, expert_counts_out, workspace,
                       workspace_bytes, path, stream);
}

int moe_forward_ep_mxfp4(const void* x, const void* Wr, const void* br, const void* Wgu_q_local,
                         const void* Wgu_s_local, const void* bgu_local, const void* Wd_q_local,
                         const void* Wd_s_local, const void* bd_local, int64_t T, int32_t H, int32_t E, int32_t k,
                         int32_t I, int32_t e_begin, int32_t n_local, float* y_partial, int32_t* topk_ids_out,
                         float* topk_w_out, void* workspace, size_t workspace_bytes, int32_t path, void* stream) {
  return forward_mxfp4("moe_forward_ep_mxfp4", x, Wr, br, Wgu_q_local, Wgu_s_local, bgu_local, Wd_q_local,
                       Wd_s_local, bd_local, T, H, E, k, I, e_begin, n_local, nullptr, y_partial, true, topk_ids_out,
                       topk_w_out, nullptr, workspace, workspace_bytes, path, stream);
}

int moe_forward_mxfp4(const void* x, const void* Wr, const void* br, const void* Wgu_q, const void* Wgu_s,
                      const void* bgu, const void* Wd_q, const void* Wd_s, const void* bd, int64_t T, int32_t H,
                      int32_t E, int32_t k, int32_t I, void* y, int32_t* topk_ids_out, float* topk_w_out,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return moe_forward_mxfp4_ex(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, T, H, E, k, I, y, topk_ids_out,
                              topk_w_out, workspace, workspace_bytes, MOE_PATH_AUTO, stream);
}

int moe_gate_up_mxfp4(const void* x, const void* Wgu_q, const void* Wgu_s, const void* bgu, const int32_t* cnt,
                      const int32_t* off, const int32_t* rows, int64_t T, int32_t H, int32_t E, int32_t k,
                      int32_t I, void* h, int32_t path, void* stream) {
  const char* fn = "moe_gate_up_mxfp4";
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  if (int st = check_mx_dims(fn, H, I)) return st;
  CHECK_PTR(x, 16);
  CHECK_PTR(Wgu_q, 16);
  CHECK_PTR(Wgu_s, 16);
  CHECK_PTR(bgu, 4);
  CHECK_PTR(cnt, 4);
  CHECK_PTR(off, 4);
  CHECK_PTR(rows, 4);
  CHECK_PTR(h, 16);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  if (int st = run_gate_up_mx(fn, x, Wgu_q, Wgu_s, bgu, cnt, off, rows, T, H, E, k, I, h, path, (hipStream_t)stream))
    return st;
  return ok();
}

int moe_down_mxfp4(const void* h, const void* Wd_q, const void* Wd_s, const void* bd, const int32_t* cnt,
                   const int32_t* off, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, float* o,
                   int32_t path, void* stream) {
  const char* fn = "moe_down_mxfp4";
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  if (int st = check_mx_dims(fn, H, I)) return st;
  CHECK_PTR(h, 16);
  CHECK_PTR(Wd_q, 16);
  CHECK_PTR(Wd_s, 16);
  CHECK_PTR(bd, 4);
  CHECK_PTR(cnt, 4);
  CHECK_PTR(off, 4);
  CHECK_PTR(o, 16);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  if (int st = run_down_mx(fn, h, Wd_q, Wd_s, bd, cnt, off, T, H, E, k, I, o, path, (hipStream_t)stream)) return st;
  return ok();
}

// ---------------------------------------------------------------------------
// FP8 W8A8
// ---------------------------------------------------------------------------
static int check_fp8_dims(const char* fn, int32_t H, int32_t I) {
  if (H % 16 != 0 || I % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: H=%d and I=%d must be multiples of 16 (16-byte code rows)", fn, H, I);
  return MOE_OK;
}

struct Fp8Layout {
  Layout base;
  size_t xq, sx, hq, sh, total;
};

static Fp8Layout fp8_layout(int64_t T, int32_t H, int32_t E, int32_t k, int32_t I) {
  Fp8Layout F;
  F.base = layout(T, H, E, k, I);
  size_t cur = F.base.total;
  const size_t S = (size_t)T * k;
  F.xq = take(cur, (size_t)T * H);
  F.sx = take(cur, (size_t)T * 4);
  F.hq = take(cur, S * I);
  F.sh = take(cur, S * 4);
  F.total = cur;
  return F;
}

size_t moe_workspace_bytes_fp8(int64_t T, int32_t H, int32_t E, int32_t k, int32_t I) {
  if (check_dims("moe_workspace_bytes_fp8", T, H, E, k, I) != MOE_OK) return 0;
  return fp8_layout(T, H, E, k, I).total;
}

int moe_quantize_fp8(const void* W, int32_t E, int32_t K, int32_t N, void* codes, float* scales, void* stream) {
  const char* fn = "moe_quantize_fp8";
  if (E < 1 || E > MOE_MAX_E) return fail(MOE_ERR_INVALID_ARG, "%s: E=%d outside [1, %d]", fn, E, MOE_MAX_E);
  if (K < 16 || K > MOE_MAX_DIM || K % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 16 in [16, %d]", fn, K, MOE_MAX_DIM);
  if (N < 8 || N > 2 * MOE_MAX_DIM || N % 8 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: N=%d must be a multiple of 8 in [8, %d]", fn, N, 2 * MOE_MAX_DIM);
  CHECK_PTR(W, 16);
  CHECK_PTR(codes, 16);
  CHECK_PTR(scales, 4);
  if (int st = hip_status(fn, moe::launch_fp8_quantize_weights(W, E, K, N, codes, scales, (hipStream_t)stream)))
    return st;
  return ok();
}

int moe_quantize_rows_fp8(const void* a, int64_t R, int32_t K, void* codes, float* scales, void* stream) {
  const char* fn = "moe_quantize_rows_fp8";
  if (R < 0) return fail(MOE_ERR_INVALID_ARG, "%s: R=%lld < 0", fn, (long long)R);
  if (K < 16 || K > MOE_MAX_DIM || K % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: K=%d must be a multiple of 16 in [16, %d]", fn, K, MOE_MAX_DIM);
  CHECK_PTR(a, 16);
  CHECK_PTR(codes, 16);
  CHECK_PTR(scales, 4);
  if (int st = hip_status(fn, moe::launch_fp8_quantize_rows(a, R, K, codes, scales, (hipStream_t)stream))) return st;
  return ok();
}

static int run_gate_up_fp8(const char* fn, const void* xq, const float* sx, const void* Wq, const float* Ws,
                           const void* bgu, const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T,
                           int32_t H, int32_t E, int32_t k, int32_t I, void* h, int32_t path, hipStream_t s) {
  path = choose_path(path, T, E, k);
  if (path == MOE_PATH_GEMM)
    return hip_status(fn, moe::launch_gemm_fp8_gate_up(xq, sx, Wq, Ws, bgu, cnt, off, rows, T, H, E, k, I, h, s));
  if (path == MOE_PATH_GEMV)
    return hip_status(fn, moe::launch_gemv_fp8_gate_up(xq, sx, Wq, Ws, bgu, cnt, off, rows, T, H, E, k, I, h, s));
  return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
}

static int run_down_fp8(const char* fn, const void* hq, const float* sh, const void* Wq, const float* Ws,
                        const void* bd, const int32_t* cnt, const int32_t* off, int64_t T, int32_t H, int32_t E,
                        int32_t k, int32_t I, float* o, int32_t path, hipStream_t s) {
  path = choose_path(path, T, E, k);
  if (path == MOE_PATH_GEMM)
    return hip_status(fn, moe::launch_gemm_fp8_down(hq, sh, Wq, Ws, bd, cnt, off, T, H, E, k, I, o, s));
  if (path == MOE_PATH_GEMV)
    return hip_status(fn, moe::launch_gemv_fp8_down(hq, sh, Wq, Ws, bd, cnt, off, T, H, E, k, I, o, s));
  return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
}

// The FP8 forward; n_valid (device, optional) marks the rows from *n_valid on
// as padding, expert_counts_out (optional) receives the per-expert loads.
static int forward_fp8(const char* fn, const void* x, const void* Wr, const void* br, const void* Wgu_q,
                       const float* Wgu_s, const void* bgu, const void* Wd_q, const float* Wd_s, const void* bd,
                       int64_t T, int32_t H, int32_t E, int32_t k, int32_t I, int32_t e_begin, int32_t n_local,
                         const int32_t* n_valid, void* y, bool partial,
                       int32_t* topk_ids_out, float* topk_w_out, int32_t* expert_counts_out, void* workspace,
                       size_t workspace_bytes, int32_t path, void* stream) {
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  if (n_local < 1 || e_begin < 0 || e_begin > E - n_local)
    return fail(MOE_ERR_INVALID_ARG, "%s: local experts [%d, %d + %d) outside [0, E=%d)", fn, e_begin, e_begin,
                n_local, E);
  if (int st = check_fp8_dims(fn, H, I)) return st;
  CHECK_PTR(x, 16);
  CHECK_PTR(Wr, 16);
  CHECK_PTR(br, 2);
  CHECK_PTR(Wgu_q, 16);
  CHECK_PTR(Wgu_s, 4);
  CHECK_PTR(bgu, 4);
  CHECK_PTR(Wd_q, 16);
  CHECK_PTR(Wd_s, 4);
  CHECK_PTR(bd, 4);
  CHECK_PTR(y, 16);
  if (topk_ids_out && !aligned(topk_ids_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_ids_out is not 4-byte aligned", fn);
  if (topk_w_out && !aligned(topk_w_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: topk_w_out is not 4-byte aligned", fn);
  if (n_valid && !aligned(n_valid, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: n_valid is not 4-byte aligned", fn);
  if (expert_counts_out && !aligned(expert_counts_out, 4))
    return fail(MOE_ERR_INVALID_ARG, "%s: expert_counts_out is not 4-byte aligned", fn);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  const Fp8Layout F = fp8_layout(T, H, E, k, I);
  if (workspace == nullptr || workspace_bytes < F.total)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, F.total);
  if (!aligned(workspace, 256))
    return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);

  char* ws = static_cast<char*>(workspace);
  const Layout& L = F.base;
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(ws + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(ws + L.w);
  int32_t* cnt = expert_counts_out ? expert_counts_out : reinterpret_cast<int32_t*>(ws + L.cnt);
  int32_t* off = reinterpret_cast<int32_t*>(ws + L.off);
  int32_t* rows = reinterpret_cast<int32_t*>(ws + L.rows);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  void* h = ws + L.h;
  float* o = reinterpret_cast<float*>(ws + L.o);
  void* xq = ws + F.xq;
  float* sx = reinterpret_cast<float*>(ws + F.sx);
  void* hq = ws + F.hq;
  float* sh = reinterpret_cast<float*>(ws + F.sh);
  hipStream_t s = (hipStream_t)stream;
  // the expert path follows the whole layer's load per expert, T*k/E
  path = choose_path(path, T, E, k);
  const int64_t S = T * k;

  if (int st = hip_status(fn, moe::launch_route(x, Wr, br, T, H, E, k, ids, w, MOE_ROUTE_AUTO, s))) return st;
  if (n_valid)
    if (int st = hip_status(fn, moe::launch_mask_padding(ids, w, T, k, n_valid, s))) return st;
  if (int st = hip_status(fn, moe::launch_permute(ids, T, n_local, k, cnt, off, rows, pos, s, e_begin))) return st;
  if (int st = hip_status(fn, moe::launch_fp8_quantize_rows(x, T, H, xq, sx, s))) return st;
  if (int st = run_gate_up_fp8(fn, xq, sx, Wgu_q, Wgu_s, bgu, cnt, off, rows, T, H, n_local, k, I, h, path, s)) return st;
  // only the rows of h the permutation filled (off[n_local] of them; fewer
  // than T*k with padding rows or on an expert-parallel rank)
  if (int st = hip_status(fn, moe::launch_fp8_quantize_rows(h, S, I, hq, sh, s, off + n_local))) return st;
  if (int st = run_down_fp8(fn, hq, sh, Wd_q, Wd_s, bd, cnt, off, T, H, n_local, k, I, o, path, s)) return st;
  if (int st = hip_status(fn, moe::launch_combine(o, pos, w, T, H, k, y, s, partial))) return st;
  return ok();
}

int moe_forward_fp8_ex(const void* x, const void* Wr, const void* br, const void* Wgu_q, const float* Wgu_s,
                       const void* bgu, const void* Wd_q, const float* Wd_s, const void* bd, int64_t T, int32_t H,
                       int32_t E, int32_t k, int32_t I, void* y, int32_t* topk_ids_out, float* topk_w_out,
                       void* workspace, size_t workspace_bytes, int32_t path, void* stream) {
  return forward_fp8("moe_forward_fp8", x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, T, H, E, k, I, 0, E,
                     nullptr, y, false, topk_ids_out, topk_w_out, nullptr, workspace, workspace_bytes, path, stream);
}

int moe_forward_padded_fp8(const void* x, const void* Wr, const void* br, const void* Wgu_q, const float* Wgu_s,
                           const void* bgu, const void* Wd_q, const float* Wd_s, const void* bd, int64_t T,
                           int32_t H, int32_t E, int32_t k, int32_t I, const int32_t* n_valid, void* y,
                           int32_t* topk_ids_out, float* topk_w_out, int32_t* expert_counts_out, void* workspace,
                           size_t workspace_bytes, int32_t path, void* stream) {
  return forward_fp8("moe_forward_padded_fp8", x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, T, H, E, k, I,
                     0, E, n_valid, y, false, topk_ids_out, topk_w_out, expert_counts_out, workspace,
                     workspace_bytes, path, stream);
}

int moe_forward_ep_fp8(const void* x, const void* Wr, const void* br, const void* Wgu_q_local,
                       const float* Wgu_s_local, const void* bgu_local, const void* Wd_q_local,
                       const float* Wd_s_local, const void* bd_local, int64_t T, int32_t H, int32_t E, int32_t k,
                       int32_t I, int32_t e_begin, int32_t n_local, float* y_partial, int32_t* topk_ids_out,
                       float* topk_w_out, void* workspace, size_t workspace_bytes, int32_t path, void* stream) {
  return forward_fp8("moe_forward_ep_fp8", x, Wr, br, Wgu_q_local, Wgu_s_local, bgu_local, Wd_q_local, Wd_s_local,
                     bd_local, T, H, E, k, I, e_begin, n_local, nullptr, y_partial, true, topk_ids_out, topk_w_out,
                     nullptr, workspace, workspace_bytes, path, stream);
}

int moe_forward_fp8(const void* x, const void* Wr, const void* br, const void* Wgu_q, const float* Wgu_s,
                    const void* bgu, const void* Wd_q, const float* Wd_s, const void* bd, int64_t T, int32_t H,
                    int32_t E, int32_t k, int32_t I, void* y, int32_t* topk_ids_out, float* topk_w_out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return moe_forward_fp8_ex(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, T, H, E, k, I, y, topk_ids_out,
                            topk_w_out, workspace, workspace_bytes, MOE_PATH_AUTO, stream);
}

int moe_gate_up_fp8(const void* xq, const float* sx, const void* Wgu_q, const float* Wgu_s, const void* bgu,
                    const int32_t* cnt, const int32_t* off, const int32_t* rows, int64_t T, int32_t H, int32_t E,
                    int32_t k, int32_t I, void* h, int32_t path, void* stream) {
  const char* fn = "moe_gate_up_fp8";
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  if (int st = check_fp8_dims(fn, H, I)) return st;
  CHECK_PTR(xq, 16);
  CHECK_PTR(sx, 4);
  CHECK_PTR(Wgu_q, 16);
  CHECK_PTR(Wgu_s, 4);
  CHECK_PTR(bgu, 4);
  CHECK_PTR(cnt, 4);
  CHECK_PTR(off, 4);
  CHECK_PTR(rows, 4);
  CHECK_PTR(h, 16);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  if (int st = run_gate_up_fp8(fn, xq, sx, Wgu_q, Wgu_s, bgu, cnt, off, rows, T, H, E, k, I, h, path,
                               (hipStream_t)stream))
    return st;
  return ok();
}

int moe_down_fp8(const void* hq, const float* sh, const void* Wd_q, const float* Wd_s, const void* bd,
                 const int32_t* cnt, const int32_t* off, int64_t T, int32_t H, int32_t E, int32_t k, int32_t I,
                 float* o, int32_t path, void* stream) {
  const char* fn = "moe_down_fp8";
  if (int st = check_dims(fn, T, H, E, k, I)) return st;
  if (int st = check_fp8_dims(fn, H, I)) return st;
  CHECK_PTR(hq, 16);
  CHECK_PTR(sh, 4);
  CHECK_PTR(Wd_q, 16);
  CHECK_PTR(Wd_s, 4);
  CHECK_PTR(bd, 4);
  CHECK_PTR(cnt, 4);
  CHECK_PTR(off, 4);
  CHECK_PTR(o, 16);
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GEMM)
    return fail(MOE_ERR_INVALID_ARG, "%s: unknown path %d", fn, path);
  if (T == 0) return ok();
  if (int st = run_down_fp8(fn, hq, sh, Wd_q, Wd_s, bd, cnt, off, T, H, E, k, I, o, path, (hipStream_t)stream))
    return st;
  return ok();
}

// ---------------------------------------------------------------------------
// measurement probes
// ---------------------------------------------------------------------------
int moe_probe_mfma_bf16(int32_t iters, int32_t workgroups, float* out, void* stream) {
  const char* fn = "moe_probe_mfma_bf16";
  if (iters < 1 || iters >= (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "%s: iters=%d outside [1, 2^20)", fn, iters);
  if (workgroups < 1 || workgroups > 65535)
    return fail(MOE_ERR_INVALID_ARG, "%s: workgroups=%d outside [1, 65535]", fn, workgroups);
  CHECK_PTR(out, 4);
  if (int st = hip_status(fn, moe::launch_probe_mfma(iters, workgroups, out, (hipStream_t)stream))) return st;
  return ok();
}

int moe_probe_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* out, void* stream) {
  const char* fn = "moe_probe_read";
  if (bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "%s: bytes=%zu is not a multiple of 16", fn, bytes);
  if (workgroups < 1 || workgroups > 65535)
    return fail(MOE_ERR_INVALID_ARG, "%s: workgroups=%d outside [1, 65535]", fn, workgroups);
  if (bytes > 0) CHECK_PTR(buf, 16);
  CHECK_PTR(out, 4);
  if (int st = hip_status(fn, moe::launch_probe_read(buf, bytes, workgroups, out, (hipStream_t)stream))) return st;
  return ok();
}

int moe_probe_mfma_dot_bf16(const void* A, const void* B, int32_t M, int32_t K, float* out, void* stream) {
  const char* fn = "moe_probe_mfma_dot_bf16";
  if (M < 16 || M % 16 != 0 || M > 16 * 65535)
    return fail(MOE_ERR_INVALID_ARG, "%s: M=%d is not a positive multiple of 16 (at most 16 * 65535)", fn, M);
  if (K < 32 || K % 32 != 0 || K > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "%s: K=%d is not a positive multiple of 32 (at most 2^20)", fn, K);
  if ((int64_t)M * K * 2 >= ((int64_t)1 << 31))
    return fail(MOE_ERR_INVALID_ARG, "%s: A of %d x %d exceeds 2 GiB", fn, M, K);
  CHECK_PTR(A, 16);
  CHECK_PTR(B, 16);
  CHECK_PTR(out, 4);
  if (int st = hip_status(fn, moe::launch_probe_dot(A, B, M, K, out, (hipStream_t)stream))) return st;
  return ok();
}

int moe_combine(const float* o, const int32_t* pos, const float* topk_w, int64_t T, int32_t H, int32_t k,
                void* y, void* stream) {
  const char* fn = "moe_combine";
  if (int st = check_dims(fn, T, H, MOE_MAX_E, k, 8)) return st;
  CHECK_PTR(o, 16);
  CHECK_PTR(pos, 4);
  CHECK_PTR(topk_w, 4);
  CHECK_PTR(y, 16);
  if (T == 0) return ok();
  if (int st = hip_status(fn, moe::launch_combine(o, pos, topk_w, T, H, k, y, (hipStream_t)stream)))
    return st;
  return ok();
}

}  // extern "C"
