// C-ABI entry points of the attention library (declared in include/fa.h): argument validation,
// workspace sizing, dispatch to the compiled kernel specialisations, and error reporting.
// Nothing here allocates device memory, and every argument error is reported before any work
// is enqueued.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <utility>

#include "fa_launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

fa_status_t fail(fa_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fa_status_t fail(fa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

fa_status_t hip_fail(hipError_t e, const char* where) {
  return fail(FA_ERR_HIP, "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxGridYZ = 65535;

fa_status_t check_common(int B, int H, int N, int d, float scale, fa_dtype_t dtype) {
  if (B <= 0 || H <= 0 || N <= 0) return fail(FA_ERR_INVALID_ARGUMENT, "B, H and N must be positive (got %d, %d, %d)", B, H, N);
  if (!std::isfinite(scale)) return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite");
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not supported (only FA_DTYPE_F32 and FA_DTYPE_BF16)", (int)dtype);
  if (d != 64 && d != 128) return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d is not supported (only 64 and 128)", d);
  if (B > kMaxGridYZ || H > kMaxGridYZ) return fail(FA_ERR_INVALID_ARGUMENT, "B and H must be at most %d", kMaxGridYZ);
  return FA_OK;
}

fa_status_t check_tensor(const void* p, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(FA_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return FA_OK;
}

fa_status_t check_f32_vec(const void* p, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned(p, 4)) return fail(FA_ERR_MISALIGNED, "%s is not 4-byte aligned", name);
  return FA_OK;
}

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

// The bf16 kernels address one head's rows through 32-bit buffer offsets.
fa_status_t check_head_bytes(int N, int d, fa_dtype_t dtype) {
  if (dtype == FA_DTYPE_BF16 && (int64_t)N * d * 2 > 0x7fffffff)
    return fail(FA_ERR_INVALID_ARGUMENT, "N*d*2 (bytes of one head) must be below 2^31 for bf16 (N=%d, d=%d)", N, d);
  return FA_OK;
}

}  // namespace

namespace fa {
BwdWorkspace bwd_workspace_layout(int B, int H, int N, int d, bool bf16) {
  BwdWorkspace w{};
  const size_t rows = (size_t)B * H * N;
  w.delta_off = 0;
  w.delta_bytes = rows * sizeof(float);
  w.lse2_off = round_up(w.delta_bytes);
  w.lse2_bytes = bf16 ? rows * sizeof(float) : 0;
  w.total = w.lse2_off + round_up(w.lse2_bytes);
  (void)d;
  return w;
}
}  // namespace fa

namespace {

fa_status_t check_workspace(int B, int H, int N, int d, fa_dtype_t dtype, const void* workspace, size_t workspace_bytes) {
  const size_t need = fa_backward_workspace_size(B, H, N, d, dtype);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0,
                need);
  if (!aligned(workspace, 16)) return fail(FA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return FA_OK;
}

fa_status_t check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  return FA_OK;
}

fa_status_t validate_prepare(const void* o, const void* dO, const float* lse, int B, int H, int N, int d,
                             fa_dtype_t dtype, void* workspace, size_t workspace_bytes) {
  fa_status_t s;
  if ((s = check_common(B, H, N, d, 0.f, dtype)) != FA_OK) return s;
  if ((s = check_tensor(o, "o")) != FA_OK || (s = check_tensor(dO, "dO")) != FA_OK ||
      (s = check_f32_vec(lse, "lse")) != FA_OK)
    return s;
  return check_workspace(B, H, N, d, dtype, workspace, workspace_bytes);
}

// Arguments shared by the two recompute stages, apart from the workspace; `outs` are the stage's outputs.
fa_status_t validate_stage_args(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                                std::initializer_list<std::pair<const void*, const char*>> outs, int B, int H, int N,
                                int d, float scale, const int32_t* seqlens, fa_dtype_t dtype) {
  fa_status_t s;
  if ((s = check_common(B, H, N, d, scale, dtype)) != FA_OK) return s;
  if ((s = check_tensor(q, "q")) != FA_OK || (s = check_tensor(k, "k")) != FA_OK || (s = check_tensor(v, "v")) != FA_OK ||
      (s = check_tensor(dO, "dO")) != FA_OK || (s = check_f32_vec(lse, "lse")) != FA_OK)
    return s;
  for (const auto& o : outs)
    if ((s = check_tensor(o.first, o.second)) != FA_OK) return s;
  if (seqlens != nullptr && !aligned(seqlens, 4)) return fail(FA_ERR_MISALIGNED, "seqlens is not 4-byte aligned");
  if (dtype == FA_DTYPE_BF16 && (fa::bwd_dkdv_bf16_grid(B, H, N) > 0x7fffffff || fa::bwd_dq_bf16_grid(B, H, N) > 0x7fffffff))
    return fail(FA_ERR_INVALID_ARGUMENT, "B*H*ceil(N/128) must be below 2^31");
  return check_head_bytes(N, d, dtype);
}

fa_status_t validate_stage(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                           std::initializer_list<std::pair<const void*, const char*>> outs, int B, int H, int N, int d,
                           float scale, const int32_t* seqlens, fa_dtype_t dtype, const void* workspace,
                           size_t workspace_bytes) {
  fa_status_t s;
  if ((s = validate_stage_args(q, k, v, dO, lse, outs, B, H, N, d, scale, seqlens, dtype)) != FA_OK) return s;
  return check_workspace(B, H, N, d, dtype, workspace, workspace_bytes);
}

fa::Problem problem(int B, int H, int N, int d, float scale, int causal, const int32_t* seqlens, void* stream) {
  return fa::Problem{B, H, N, d, scale, causal != 0, seqlens, (hipStream_t)stream};
}

fa_status_t run_prepare(const fa::Problem& p, fa_dtype_t dtype, const void* o, const void* dO, const float* lse,
                        void* workspace) {
  hipError_t e = fa::launch_bwd_prepare(p, dtype == FA_DTYPE_BF16, o, dO, lse, workspace);
  return e == hipSuccess ? FA_OK : hip_fail(e, "backward prepare launch");
}

fa_status_t run_dkdv(const fa::Problem& p, fa_dtype_t dtype, const void* q, const void* k, const void* v,
                     const void* dO, const float* lse, void* dk, void* dv, const void* workspace) {
  hipError_t e = (dtype == FA_DTYPE_BF16)
                     ? fa::launch_bwd_dkdv_bf16(p, q, k, v, dO, dk, dv, workspace)
                     : fa::launch_bwd_dkdv_f32(p, (const float*)q, (const float*)k, (const float*)v, (const float*)dO,
                                               lse, (float*)dk, (float*)dv, workspace);
  return e == hipSuccess ? FA_OK : hip_fail(e, "backward dK/dV launch");
}

fa_status_t run_dq(const fa::Problem& p, fa_dtype_t dtype, const void* q, const void* k, const void* v,
                   const void* dO, const float* lse, void* dq, const void* workspace) {
  hipError_t e = (dtype == FA_DTYPE_BF16)
                     ? fa::launch_bwd_dq_bf16(p, q, k, v, dO, dq, workspace)
                     : fa::launch_bwd_dq_f32(p, (const float*)q, (const float*)k, (const float*)v, (const float*)dO,
                                             lse, (float*)dq, workspace);
  return e == hipSuccess ? FA_OK : hip_fail(e, "backward dQ launch");
}

// The dQ pass with the prepare stage folded in (bf16): also writes -D and LSE log2(e) into the workspace.
fa_status_t run_dq_prepare(fa::Problem p, const void* q, const void* k, const void* v, const void* o, const void* dO,
                           const float* lse, void* dq, void* workspace) {
  p.pre_o = o;
  p.pre_lse = lse;
  hipError_t e = fa::launch_bwd_dq_bf16(p, q, k, v, dO, dq, workspace);
  return e == hipSuccess ? FA_OK : hip_fail(e, "backward dQ (with prepare) launch");
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE";
    case FA_ERR_HIP: return "FA_ERR_HIP";
  }
  return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error; }

size_t fa_backward_workspace_size(int B, int H, int N, int d, fa_dtype_t dtype) {
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128) || (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16)) return 0;
  return fa::bwd_workspace_layout(B, H, N, d, dtype == FA_DTYPE_BF16).total;
}

}  // extern "C"

namespace {

fa_status_t check_block_mask(const uint8_t* block_mask, int N) {
  if (block_mask == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "block_mask is NULL");
  if (N > FA_MASK_MAX_N)
    return fail(FA_ERR_UNSUPPORTED, "block-sparse attention supports N <= %d (got %d)", FA_MASK_MAX_N, N);
  return FA_OK;
}

// Dropout parameters of a call (none: p < 0 is never passed by the entry points that have no dropout).
struct DropArgs {
  bool on = false;
  float p = 0.f;
  uint64_t seed = 0;
  uint32_t offset = 0;
};

fa_status_t check_dropout(float p, int* t) {
  if (!std::isfinite(p) || p < 0.f) return fail(FA_ERR_INVALID_ARGUMENT, "dropout_p must be finite and >= 0");
  const double x = std::nearbyint((1.0 - (double)p) * 256.0);  // half to even
  if (x < 1.0 || x > 256.0)
    return fail(FA_ERR_INVALID_ARGUMENT, "dropout_p=%g leaves no kept element (round((1-p)*256) < 1)", (double)p);
  *t = (int)x;
  return FA_OK;
}

void set_dropout(fa::Problem& pr, const DropArgs& dr, int t) {
  pr.dropout = dr.on;
  pr.drop_k0 = (uint32_t)dr.seed;
  pr.drop_k1 = (uint32_t)(dr.seed >> 32);
  pr.drop_off2 = 2u * dr.offset;
  pr.drop_t = (uint32_t)t;
}

fa_status_t forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                         float scale, int causal, const int32_t* seqlens, const uint8_t* block_mask, fa_dtype_t dtype,
                         void* stream, const DropArgs& drop = DropArgs()) {
  fa_status_t s;
  if ((s = check_common(B, H, N, d, scale, dtype)) != FA_OK) return s;
  if ((s = check_tensor(q, "q")) != FA_OK || (s = check_tensor(k, "k")) != FA_OK || (s = check_tensor(v, "v")) != FA_OK ||
      (s = check_tensor(o, "o")) != FA_OK || (s = check_f32_vec(lse, "lse")) != FA_OK)
    return s;
  if (seqlens != nullptr && !aligned(seqlens, 4)) return fail(FA_ERR_MISALIGNED, "seqlens is not 4-byte aligned");
  if (dtype == FA_DTYPE_BF16 && fa::fwd_bf16_grid(B, H, N) > 0x7fffffff)
    return fail(FA_ERR_INVALID_ARGUMENT, "B*H*ceil(N/128) must be below 2^31");
  if ((s = check_head_bytes(N, d, dtype)) != FA_OK) return s;
  int t = 256;
  if (drop.on && (s = check_dropout(drop.p, &t)) != FA_OK) return s;
  if ((s = check_device()) != FA_OK) return s;
  fa::Problem p = problem(B, H, N, d, scale, causal, seqlens, stream);
  p.block_mask = block_mask;
  set_dropout(p, drop, t);
  const hipError_t e = (dtype == FA_DTYPE_BF16) ? fa::launch_fwd_bf16(p, q, k, v, o, lse)
                               : fa::launch_fwd_f32(p, (const float*)q, (const float*)k, (const float*)v, (float*)o, lse);
  if (e != hipSuccess) return hip_fail(e, "fa_forward launch");
  return FA_OK;
}

fa_status_t backward_impl(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                          void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                          const int32_t* seqlens, const uint8_t* block_mask, fa_dtype_t dtype, void* workspace,
                          size_t workspace_bytes, void* stream, const DropArgs& drop = DropArgs()) {
  fa_status_t s;
  if ((s = validate_stage(q, k, v, dO, lse, {{dq, "dq"}, {dk, "dk"}, {dv, "dv"}}, B, H, N, d, scale, seqlens, dtype,
                          workspace, workspace_bytes)) != FA_OK)
    return s;
  if ((s = check_tensor(o, "o")) != FA_OK) return s;
  int t = 256;
  if (drop.on && (s = check_dropout(drop.p, &t)) != FA_OK) return s;
  if ((s = check_device()) != FA_OK) return s;
  fa::Problem p = problem(B, H, N, d, scale, causal, seqlens, stream);
  p.block_mask = block_mask;
  set_dropout(p, drop, t);
  if (dtype == FA_DTYPE_BF16) {
    // bf16: the dQ pass forms the row statistics itself (every query row has its dQ workgroup, whatever
    // the block mask or dropout), then the dK/dV pass reads them
    if ((s = run_dq_prepare(p, q, k, v, o, dO, lse, dq, workspace)) != FA_OK) return s;
    return run_dkdv(p, dtype, q, k, v, dO, lse, dk, dv, workspace);
  }
  if ((s = run_prepare(p, dtype, o, dO, lse, workspace)) != FA_OK) return s;
  if ((s = run_dkdv(p, dtype, q, k, v, dO, lse, dk, dv, workspace)) != FA_OK) return s;
  return run_dq(p, dtype, q, k, v, dO, lse, dq, workspace);
}

}  // namespace

extern "C" {

fa_status_t fa_forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                       float scale, int causal, const int32_t* seqlens, fa_dtype_t dtype, void* stream) {
  g_last_error[0] = '\0';
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, seqlens, nullptr, dtype, stream);
}

fa_status_t fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                    int N, int d, float scale, int causal, const int32_t* seqlens,
                                    const uint8_t* block_mask, fa_dtype_t dtype, void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = check_block_mask(block_mask, N)) != FA_OK) return s;
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, seqlens, block_mask, dtype, stream);
}

fa_status_t fa_backward(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                        void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                        const int32_t* seqlens, fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                        void* stream) {
  g_last_error[0] = '\0';
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, seqlens, nullptr, dtype, workspace,
                       workspace_bytes, stream);
}

fa_status_t fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                               int d, float scale, int causal, const int32_t* seqlens, float dropout_p, uint64_t seed,
                               uint32_t offset, fa_dtype_t dtype, void* stream) {
  g_last_error[0] = '\0';
  DropArgs dr;
  dr.on = true;
  dr.p = dropout_p;
  dr.seed = seed;
  dr.offset = offset;
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, seqlens, nullptr, dtype, stream, dr);
}

fa_status_t fa_backward_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                                int causal, const int32_t* seqlens, float dropout_p, uint64_t seed, uint32_t offset,
                                fa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  DropArgs dr;
  dr.on = true;
  dr.p = dropout_p;
  dr.seed = seed;
  dr.offset = offset;
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, seqlens, nullptr, dtype, workspace,
                       workspace_bytes, stream, dr);
}

fa_status_t fa_dropout_mask(int B, int H, int N, float dropout_p, uint64_t seed, uint32_t offset, uint8_t* keep,
                            void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if (B <= 0 || H <= 0 || N <= 0) return fail(FA_ERR_INVALID_ARGUMENT, "B, H and N must be positive (got %d, %d, %d)", B, H, N);
  if (keep == nullptr) return fail(FA_ERR_INVALID_ARGUMENT, "keep is NULL");
  const int64_t total = (int64_t)B * H * N * ((N + 31) / 32);
  if ((total + 255) / 256 > 0x7fffffff) return fail(FA_ERR_INVALID_ARGUMENT, "B*H*N*ceil(N/32) too large");
  int t = 256;
  if ((s = check_dropout(dropout_p, &t)) != FA_OK) return s;
  if ((s = check_device()) != FA_OK) return s;
  fa::Problem p = problem(B, H, N, 64, 1.f, 0, nullptr, stream);
  DropArgs dr;
  dr.on = true;
  dr.p = dropout_p;
  dr.seed = seed;
  dr.offset = offset;
  set_dropout(p, dr, t);
  const hipError_t e = fa::launch_dropout_mask(p, keep);
  return e == hipSuccess ? FA_OK : hip_fail(e, "fa_dropout_mask launch");
}

fa_status_t fa_forward_fp8(const void* q8, const void* k8, const void* v8, float descale_q, float descale_k,
                           float descale_v, void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
                           const int32_t* seqlens, void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = check_common(B, H, N, d, scale, FA_DTYPE_BF16)) != FA_OK) return s;
  if (d != 128) return fail(FA_ERR_UNSUPPORTED, "the FP8 forward supports d = 128 only (got %d)", d);
  for (float x : {descale_q, descale_k, descale_v})
    if (!std::isfinite(x) || !(x > 0.f)) return fail(FA_ERR_INVALID_ARGUMENT, "descales must be finite and positive");
  if ((s = check_tensor(q8, "q8")) != FA_OK || (s = check_tensor(k8, "k8")) != FA_OK ||
      (s = check_tensor(v8, "v8")) != FA_OK || (s = check_tensor(o, "o")) != FA_OK ||
      (s = check_f32_vec(lse, "lse")) != FA_OK)
    return s;
  if (seqlens != nullptr && !aligned(seqlens, 4)) return fail(FA_ERR_MISALIGNED, "seqlens is not 4-byte aligned");
  if (fa::fwd_bf16_grid(B, H, N) > 0x7fffffff) return fail(FA_ERR_INVALID_ARGUMENT, "B*H*ceil(N/128) must be below 2^31");
  if ((s = check_head_bytes(N, d, FA_DTYPE_BF16)) != FA_OK) return s;
  if ((s = check_device()) != FA_OK) return s;
  fa::Problem p = problem(B, H, N, d, scale, causal, seqlens, stream);
  p.fp8_qk_descale = descale_q * descale_k;
  p.fp8_v_descale = descale_v;
  const hipError_t e = fa::launch_fwd_fp8(p, q8, k8, v8, o, lse);
  return e == hipSuccess ? FA_OK : hip_fail(e, "fa_forward_fp8 launch");
}

size_t fa_forward_kv_outer_workspace_size(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || (d != 64 && d != 128)) return 0;
  const size_t rows = (size_t)B * H * N;
  return rows * (size_t)d * 4 + 2 * rows * 4;
}

fa_status_t fa_forward_kv_outer(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                                int d, float scale, size_t lds_bytes, fa_dtype_t dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = check_common(B, H, N, d, scale, dtype)) != FA_OK) return s;
  if (dtype != FA_DTYPE_BF16) return fail(FA_ERR_UNSUPPORTED, "the K/V-outer schedule takes bf16 inputs only");
  if ((s = check_tensor(q, "q")) != FA_OK || (s = check_tensor(k, "k")) != FA_OK || (s = check_tensor(v, "v")) != FA_OK ||
      (s = check_tensor(o, "o")) != FA_OK || (s = check_f32_vec(lse, "lse")) != FA_OK)
    return s;
  if ((int64_t)B * H > 0x7fffffff) return fail(FA_ERR_INVALID_ARGUMENT, "B*H must be below 2^31");
  const fa::KvOuterTiles t = fa::kv_outer_tiles(d, lds_bytes);
  if (lds_bytes == 0 || t.Bc < 1 || t.smem > 160 * 1024)
    return fail(FA_ERR_UNSUPPORTED, "LDS budget of %zu bytes gives tiles B_c=%d, B_r=%d needing %zu bytes (at most 160 KiB)",
                lds_bytes, t.Bc, t.Br, t.smem);
  const size_t need = fa_forward_kv_outer_workspace_size(B, H, N, d);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : (size_t)0, need);
  if (!aligned(workspace, 16)) return fail(FA_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  if ((s = check_device()) != FA_OK) return s;
  const fa::Problem p = problem(B, H, N, d, scale, 0, nullptr, stream);
  const hipError_t e = fa::launch_fwd_kv_outer(p, q, k, v, o, lse, workspace, lds_bytes);
  return e == hipSuccess ? FA_OK : hip_fail(e, "fa_forward_kv_outer launch");
}

fa_status_t fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                     float scale, int causal, const int32_t* seqlens, const uint8_t* block_mask,
                                     fa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = check_block_mask(block_mask, N)) != FA_OK) return s;
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, seqlens, block_mask, dtype,
                       workspace, workspace_bytes, stream);
}

fa_status_t fa_backward_prepare(const void* o, const void* dO, const float* lse, int B, int H, int N, int d,
                                fa_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = validate_prepare(o, dO, lse, B, H, N, d, dtype, workspace, workspace_bytes)) != FA_OK) return s;
  if ((s = check_device()) != FA_OK) return s;
  return run_prepare(problem(B, H, N, d, 1.f, 0, nullptr, stream), dtype, o, dO, lse, workspace);
}

fa_status_t fa_backward_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dk,
                             void* dv, int B, int H, int N, int d, float scale, int causal, const int32_t* seqlens,
                             fa_dtype_t dtype, const void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = validate_stage(q, k, v, dO, lse, {{dk, "dk"}, {dv, "dv"}}, B, H, N, d, scale, seqlens, dtype, workspace,
                          workspace_bytes)) != FA_OK)
    return s;
  if ((s = check_device()) != FA_OK) return s;
  return run_dkdv(problem(B, H, N, d, scale, causal, seqlens, stream), dtype, q, k, v, dO, lse, dk, dv, workspace);
}

fa_status_t fa_backward_dq_prepare(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                   const float* lse, void* dq, int B, int H, int N, int d, float scale, int causal,
                                   const int32_t* seqlens, fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = validate_stage(q, k, v, dO, lse, {{dq, "dq"}}, B, H, N, d, scale, seqlens, dtype, workspace,
                          workspace_bytes)) != FA_OK)
    return s;
  if ((s = check_tensor(o, "o")) != FA_OK) return s;
  if ((s = check_device()) != FA_OK) return s;
  const fa::Problem p = problem(B, H, N, d, scale, causal, seqlens, stream);
  if (dtype == FA_DTYPE_BF16) return run_dq_prepare(p, q, k, v, o, dO, lse, dq, workspace);
  if ((s = run_prepare(p, dtype, o, dO, lse, workspace)) != FA_OK) return s;
  return run_dq(p, dtype, q, k, v, dO, lse, dq, workspace);
}

fa_status_t fa_backward_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse, void* dq,
                           int B, int H, int N, int d, float scale, int causal, const int32_t* seqlens,
                           fa_dtype_t dtype, const void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = validate_stage(q, k, v, dO, lse, {{dq, "dq"}}, B, H, N, d, scale, seqlens, dtype, workspace,
                          workspace_bytes)) != FA_OK)
    return s;
  if ((s = check_device()) != FA_OK) return s;
  return run_dq(problem(B, H, N, d, scale, causal, seqlens, stream), dtype, q, k, v, dO, lse, dq, workspace);
}

}  // extern "C"

// ---- fa_backward_noalloc: the backward with a workspace the library holds itself, for callers that
// cannot allocate device memory.  The workspace is a file-scope device array (one copy per GPU,
// alive until the process ends).  In host code the array's name is only a stand-in: its device
// address, which differs per GPU, comes from hipGetSymbolAddress on the first call with that
// device current, and only that address is ever passed to a kernel.
namespace {

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (resolved once per device).
fa_status_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(FA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status_t fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                                const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                float scale, int causal, const int32_t* seqlens, fa_dtype_t dtype, void* stream) {
  g_last_error[0] = '\0';
  fa_status_t s;
  if ((s = check_common(B, H, N, d, scale, dtype)) != FA_OK) return s;
  const size_t need = fa_backward_workspace_size(B, H, N, d, dtype);
  if (need > (size_t)FA_NOALLOC_WORKSPACE_BYTES)
    return fail(FA_ERR_UNSUPPORTED,
                "fa_backward_noalloc: B*H*N = %lld rows need %zu bytes of workspace, more than its %d; use fa_backward",
                (long long)B * H * N, need, FA_NOALLOC_WORKSPACE_BYTES);
  // every other argument is validated as for fa_backward before the device is asked for the workspace,
  // so an argument error is reported without any device call
  if ((s = validate_stage_args(q, k, v, dO, lse, {{dq, "dq"}, {dk, "dk"}, {dv, "dv"}}, B, H, N, d, scale, seqlens,
                               dtype)) != FA_OK)
    return s;
  if ((s = check_tensor(o, "o")) != FA_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != FA_OK) return s;
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, seqlens, nullptr, dtype, ws, need,
                       stream);
}

}  // extern "C"
