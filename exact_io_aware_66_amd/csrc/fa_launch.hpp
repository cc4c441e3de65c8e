// Host-side launchers of the attention kernels (internal to the library; the public ABI is fa.h).
// Each launcher assumes its arguments were validated by the C-ABI layer and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct Problem {
  int B, H, N, d;
  float scale;
  bool causal;
  const int32_t* seqlens;  // device int32[B] or nullptr
  hipStream_t stream;
  const uint8_t* block_mask = nullptr;  // device uint8[B][H][nb][nb] (nb = ceil(N/128)), or nullptr: dense
  bool dropout = false;                 // dropout on the attention probabilities (dense attention only)
  uint32_t drop_k0 = 0, drop_k1 = 0;    // Philox key: seed low and high words
  uint32_t drop_off2 = 0;               // 2 offset
  uint32_t drop_t = 256;                // keep threshold round((1 - p) 256)
  float fp8_qk_descale = 1.f;           // FP8 forward: descale(Q) descale(K), folded into the score scale
  float fp8_v_descale = 1.f;            // FP8 forward: descale(V), applied to O
  // dQ pass that also forms the row statistics (the prepare stage folded in): O and the forward's
  // LSE, or nullptr when the workspace already holds D and LSE log2(e)
  const void* pre_o = nullptr;
  const float* pre_lse = nullptr;
};

// Workspace carve-up of the backward (byte offsets; all 256-byte aligned).
struct BwdWorkspace {
  size_t delta_off, delta_bytes;  // float32 [B][H][N]: D_i = sum_c dO_ic O_ic
  size_t lse2_off, lse2_bytes;    // float32 [B][H][N]: LSE_i log2(e) (bf16 path only)
  size_t total;
};
BwdWorkspace bwd_workspace_layout(int B, int H, int N, int d, bool bf16);

// Workgroups of the bf16 launches (each one 1-D grid over row blocks x B x H).
int64_t fwd_bf16_grid(int B, int H, int N);
int64_t bwd_dkdv_bf16_grid(int B, int H, int N);
int64_t bwd_dq_bf16_grid(int B, int H, int N);

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse);
// Forward with OCP FP8 E4M3 inputs (d = 128): S on the FP8 matrix cores, P V in bf16.
hipError_t launch_fwd_fp8(const Problem& p, const void* q8, const void* k8, const void* v8, void* o, float* lse);
hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o, float* lse);
// Backward stages.  prepare: D (and, for bf16, LSE log2 e) into the workspace; dkdv: dK and dV;
// dq: dQ.  dkdv and dq read the workspace that prepare wrote and are independent of each other; a dQ
// launch with p.pre_o set writes that workspace itself (so it must precede dkdv).
hipError_t launch_bwd_prepare(const Problem& p, bool bf16, const void* o, const void* dO, const float* lse,
                              void* workspace);
hipError_t launch_bwd_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                                void* dk, void* dv, const void* workspace);
// dK/dV at d = 128 without a block mask (dense or with dropout) with K in LDS and two waves per SIMD
// (bitwise the results of the general kernel; lse2: LSE log2(e), ndelta: -D, both from the workspace).
hipError_t launch_dkdv_kl_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                               const float* lse2, const float* ndelta, void* dk, void* dv);
// With p.pre_o set, the dQ pass also writes D and LSE log2(e) of its rows into the workspace, bitwise equal
// to what launch_bwd_prepare writes.
hipError_t launch_bwd_dq_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO, void* dq,
                              const void* workspace);
hipError_t launch_bwd_dkdv_f32(const Problem& p, const float* q, const float* k, const float* v, const float* dO,
                               const float* lse, float* dk, float* dv, const void* workspace);
// The pages' K/V-outer schedule (IO-complexity measurement): tiles from an LDS budget of lds_bytes
// (fp32 elements), workspace = fp32 O [B][H][N][d], m and l [B][H][N].
struct KvOuterTiles {
  int Bc, Br;
  size_t smem;  // LDS bytes the kernel uses for these tiles (K, V, Q, O tiles, S, two row factors)
};
KvOuterTiles kv_outer_tiles(int d, size_t lds_bytes);
hipError_t launch_fwd_kv_outer(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse,
                               void* workspace, size_t lds_bytes);
// Dropout keep mask as bytes (1 = kept), [B][H][N][N]: the decisions every kernel takes.
hipError_t launch_dropout_mask(const Problem& p, uint8_t* keep);
hipError_t launch_bwd_dq_f32(const Problem& p, const float* q, const float* k, const float* v, const float* dO,
                             const float* lse, float* dq, const void* workspace);

}  // namespace fa
