// Host-side launchers of the attention kernels (internal to the library; the public ABI is fa.h).
// Each launcher assumes its arguments were validated by the C-ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifndef FA_FWD_ROWS_PER_WAVE
#define FA_FWD_ROWS_PER_WAVE 32  // query rows per wave of the bf16 forward kernel (32 or 64)
#endif

namespace fa {

struct Problem {
  int B, H, N, d;
  float scale;
  bool causal;
  const int32_t* seqlens;  // device int32[B] or nullptr
  hipStream_t stream;
};

// Workspace carve-up of the backward (byte offsets; all 256-byte aligned).
struct BwdWorkspace {
  size_t delta_off, delta_bytes;  // float32 [B][H][N]: D_i = sum_c dO_ic O_ic
  size_t lse2_off, lse2_bytes;    // float32 [B][H][N]: LSE_i log2(e) (bf16 path only)
  size_t dqacc_off, dqacc_bytes;  // float32 [B][H][Npad][d] dQ accumulator, rows padded (bf16 path only)
  size_t total;
};
BwdWorkspace bwd_workspace_layout(int B, int H, int N, int d, bool bf16);
// Rows per head of the bf16 dQ accumulator (N rounded up to the backward's query tile).
int bwd_rows_padded(int N);
// Workgroups of the bf16 backward main launch.
int64_t bwd_bf16_grid(int B, int H, int N);

// Workgroups of the bf16 forward launch (one 1-D grid over query blocks x B x H).
int64_t fwd_bf16_grid(int B, int H, int N);
hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse);
hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o, float* lse);
// Backward stages.  prepare: D (and, for bf16, LSE log2 e and a cleared dQ accumulator); main: dK, dV and dQ
// accumulation; finish (bf16 only): dq = bf16(scale * accumulator).
hipError_t launch_bwd_prepare(const Problem& p, bool bf16, const void* o, const void* dO, const float* lse,
                              void* workspace);
hipError_t launch_bwd_main_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                                void* dk, void* dv, void* workspace);
hipError_t launch_bwd_finish_bf16(const Problem& p, void* dq, void* workspace);
hipError_t launch_bwd_main_f32(const Problem& p, const float* q, const float* k, const float* v, const float* dO,
                               const float* lse, float* dq, float* dk, float* dv, void* workspace);

}  // namespace fa
