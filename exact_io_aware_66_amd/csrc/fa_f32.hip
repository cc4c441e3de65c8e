// Exact attention for float32 inputs (forward and backward) on the gfx950 vector ALUs.
//
// The same tiled, fused algorithm as the bf16 path -- key/value (or query) tiles staged in LDS,
// online softmax with a running maximum and normaliser per row, the backward recomputing P from
// the stored log-sum-exp (NOTE-005: FlashAttention, "Method") -- but every product is an fp32 FMA
// and every row is owned by one thread.  gfx950 has no fp32-input matrix-core shortcut of useful
// precision, and this path exists for exact fp32 results at small sizes, not for throughput.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kF32Rows = 64;  // rows (threads) per workgroup
constexpr int kF32Tile = 32;  // staged rows per LDS tile

// Visibility of key `key` to query `query` (keys >= L are padding; causal keeps key <= query).
template <bool CAUSAL>
__device__ __forceinline__ bool visible(int query, int key, int L) {
  return key < L && (!CAUSAL || key <= query);
}

// Block-sparse: whether mask block (query row r, key column c) of head bh is visible (always, when
// there is no block mask).  Workgroups (64 rows) and tiles (32 rows) never straddle a 128 x 128
// block, so one lookup decides a whole tile for the whole workgroup.
__device__ __forceinline__ bool block_visible(const uint8_t* bmask, int64_t bh, int N, int r, int c) {
  if (bmask == nullptr) return true;
  const int nb = (N + kMaskBlock - 1) / kMaskBlock;
  return bmask[(bh * nb + r / kMaskBlock) * nb + c / kMaskBlock] != 0;
}

// ---------------------------------------------------------------------------------------------
// Forward: thread = query row; K/V tiles of 32 keys in LDS; per tile the 32 scores are formed,
// the running max/normaliser updated once, and the output rescaled once.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, float* __restrict__ O,
                                                     float* __restrict__ LSE, int H, int N, float scale,
                                                     const int32_t* __restrict__ seqlens,
                                                     const uint8_t* __restrict__ bmask) {
  __shared__ float ks[kF32Tile][D];
  __shared__ float vs[kF32Tile][D];
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t row0 = ((int64_t)b * H + h) * N;
  const int L = seqlens ? clamp_len(seqlens, b, N) : N;
  const int q0 = blockIdx.x * kF32Rows;
  const int query = q0 + threadIdx.x;
  const int qrow = min(query, N - 1);
  float q[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = Q[(row0 + qrow) * D + c];
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  int kend = L;
  if (CAUSAL) kend = min(kend, q0 + kF32Rows);
  for (int k0 = 0; k0 < kend; k0 += kF32Tile) {
    if (!block_visible(bmask, (int64_t)b * H + h, N, q0, k0)) continue;
    __syncthreads();
    for (int i = threadIdx.x; i < kF32Tile * D; i += 64) {
      const int r = i / D, c = i % D;
      const int key = min(k0 + r, N - 1);
      ks[r][c] = K[(row0 + key) * D + c];
      vs[r][c] = V[(row0 + key) * D + c];
    }
    __syncthreads();
    float s[kF32Tile];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Tile; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(q[c], ks[j][c], dot);
      s[j] = visible<CAUSAL>(query, k0 + j, L) ? dot * scale : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m - m_use);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32Tile; ++j) {
      const float p = expf(s[j] - m_use);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vs[j][c], acc[c]);
    }
    m = m_new;
  }
  if (query < N) {
    const bool has = l > 0.f;
    const float inv = has ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) O[(row0 + query) * D + c] = acc[c] * inv;
    LSE[row0 + query] = has ? m + logf(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------------
// Backward, dK and dV: thread = key row (its K and V rows staged in LDS), loop over query tiles.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void bwd_kv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V, const float* __restrict__ dO,
                                                        const float* __restrict__ LSE, const float* __restrict__ DELTA,
                                                        float* __restrict__ dK, float* __restrict__ dV, int H, int N,
                                                        float scale, const int32_t* __restrict__ seqlens,
                                                        const uint8_t* __restrict__ bmask) {
  __shared__ float kr[kF32Rows][D + 1];
  __shared__ float vr[kF32Rows][D + 1];
  __shared__ float qs[kF32Tile][D];
  __shared__ float gs[kF32Tile][D];
  __shared__ float lse_s[kF32Tile], del_s[kF32Tile];
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t row0 = ((int64_t)b * H + h) * N;
  const int L = seqlens ? clamp_len(seqlens, b, N) : N;
  const int k0 = blockIdx.x * kF32Rows;
  const int key = k0 + threadIdx.x;
  for (int i = threadIdx.x; i < kF32Rows * D; i += 64) {
    const int r = i / D, c = i % D;
    const int kk = min(k0 + r, N - 1);
    kr[r][c] = K[(row0 + kk) * D + c];
    vr[r][c] = V[(row0 + kk) * D + c];
  }
  float dk[D], dv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    dk[c] = 0.f;
    dv[c] = 0.f;
  }
  const int qstart = CAUSAL ? k0 : 0;
  const int qtile0 = (k0 < L) ? (qstart / kF32Tile) * kF32Tile : N;  // no visible key: skip the walk
  for (int qt0 = qtile0; qt0 < N; qt0 += kF32Tile) {
    if (!block_visible(bmask, (int64_t)b * H + h, N, qt0, k0)) continue;
    __syncthreads();
    for (int i = threadIdx.x; i < kF32Tile * D; i += 64) {
      const int r = i / D, c = i % D;
      const int qq = min(qt0 + r, N - 1);
      qs[r][c] = Q[(row0 + qq) * D + c];
      gs[r][c] = dO[(row0 + qq) * D + c];
    }
    if (threadIdx.x < kF32Tile) {
      const int qq = min(qt0 + (int)threadIdx.x, N - 1);
      lse_s[threadIdx.x] = LSE[row0 + qq];
      del_s[threadIdx.x] = DELTA[row0 + qq];
    }
    __syncthreads();
    for (int i = 0; i < kF32Tile; ++i) {
      const int query = qt0 + i;
      if (query >= N || !visible<CAUSAL>(query, key, L)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = fmaf(qs[i][c], kr[threadIdx.x][c], s);
        dp = fmaf(gs[i][c], vr[threadIdx.x][c], dp);
      }
      const float p = expf(s * scale - lse_s[i]);
      const float dsv = p * (dp - del_s[i]);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        dv[c] = fmaf(p, gs[i][c], dv[c]);
        dk[c] = fmaf(dsv, qs[i][c], dk[c]);
      }
    }
  }
  if (key < N) {
#pragma unroll
    for (int c = 0; c < D; ++c) {
      dK[(row0 + key) * D + c] = dk[c] * scale;
      dV[(row0 + key) * D + c] = dv[c];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Backward, dQ: thread = query row (its Q and dO rows staged in LDS), loop over key tiles.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void bwd_q_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       const float* __restrict__ LSE, const float* __restrict__ DELTA,
                                                       float* __restrict__ dQ, int H, int N, float scale,
                                                       const int32_t* __restrict__ seqlens,
                                                       const uint8_t* __restrict__ bmask) {
  __shared__ float qr[kF32Rows][D + 1];
  __shared__ float gr[kF32Rows][D + 1];
  __shared__ float ks[kF32Tile][D];
  __shared__ float vs[kF32Tile][D];
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t row0 = ((int64_t)b * H + h) * N;
  const int L = seqlens ? clamp_len(seqlens, b, N) : N;
  const int q0 = blockIdx.x * kF32Rows;
  const int query = q0 + threadIdx.x;
  const int qrow = min(query, N - 1);
  for (int i = threadIdx.x; i < kF32Rows * D; i += 64) {
    const int r = i / D, c = i % D;
    const int qq = min(q0 + r, N - 1);
    qr[r][c] = Q[(row0 + qq) * D + c];
    gr[r][c] = dO[(row0 + qq) * D + c];
  }
  const float lse = LSE[row0 + qrow];
  const float del = DELTA[row0 + qrow];
  float dq[D];
#pragma unroll
  for (int c = 0; c < D; ++c) dq[c] = 0.f;
  int kend = L;
  if (CAUSAL) kend = min(kend, q0 + kF32Rows);
  for (int k0 = 0; k0 < kend; k0 += kF32Tile) {
    if (!block_visible(bmask, (int64_t)b * H + h, N, q0, k0)) continue;
    __syncthreads();
    for (int i = threadIdx.x; i < kF32Tile * D; i += 64) {
      const int r = i / D, c = i % D;
      const int kk = min(k0 + r, N - 1);
      ks[r][c] = K[(row0 + kk) * D + c];
      vs[r][c] = V[(row0 + kk) * D + c];
    }
    __syncthreads();
    for (int j = 0; j < kF32Tile; ++j) {
      if (!visible<CAUSAL>(query, k0 + j, L)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = fmaf(qr[threadIdx.x][c], ks[j][c], s);
        dp = fmaf(gr[threadIdx.x][c], vs[j][c], dp);
      }
      const float p = expf(s * scale - lse);
      const float dsv = p * (dp - del);
#pragma unroll
      for (int c = 0; c < D; ++c) dq[c] = fmaf(dsv, ks[j][c], dq[c]);
    }
  }
  if (query < N) {
#pragma unroll
    for (int c = 0; c < D; ++c) dQ[(row0 + query) * D + c] = dq[c] * scale;
  }
}

template <int D, bool CAUSAL>
hipError_t fwd(const Problem& p, const float* q, const float* k, const float* v, float* o, float* lse) {
  dim3 grid((p.N + kF32Rows - 1) / kF32Rows, p.H, p.B);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), grid, dim3(64), 0, p.stream, q, k, v, o, lse, p.H, p.N, p.scale,
                     p.seqlens, p.block_mask);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t bwd_kv(const Problem& p, const float* q, const float* k, const float* v, const float* dO, const float* lse,
                  const float* delta, float* dk, float* dv) {
  dim3 grid((p.N + kF32Rows - 1) / kF32Rows, p.H, p.B);
  hipLaunchKernelGGL((bwd_kv_f32_kernel<D, CAUSAL>), grid, dim3(64), 0, p.stream, q, k, v, dO, lse, delta, dk, dv,
                     p.H, p.N, p.scale, p.seqlens, p.block_mask);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t bwd_q(const Problem& p, const float* q, const float* k, const float* v, const float* dO, const float* lse,
                 const float* delta, float* dq) {
  dim3 grid((p.N + kF32Rows - 1) / kF32Rows, p.H, p.B);
  hipLaunchKernelGGL((bwd_q_f32_kernel<D, CAUSAL>), grid, dim3(64), 0, p.stream, q, k, v, dO, lse, delta, dq, p.H,
                     p.N, p.scale, p.seqlens, p.block_mask);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o, float* lse) {
  if (p.d == 64) return p.causal ? fwd<64, true>(p, q, k, v, o, lse) : fwd<64, false>(p, q, k, v, o, lse);
  return p.causal ? fwd<128, true>(p, q, k, v, o, lse) : fwd<128, false>(p, q, k, v, o, lse);
}

hipError_t launch_bwd_dkdv_f32(const Problem& p, const float* q, const float* k, const float* v, const float* dO,
                               const float* lse, float* dk, float* dv, const void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, false);
  const float* delta = (const float*)((const char*)workspace + ws.delta_off);
  if (p.d == 64)
    return p.causal ? bwd_kv<64, true>(p, q, k, v, dO, lse, delta, dk, dv)
                    : bwd_kv<64, false>(p, q, k, v, dO, lse, delta, dk, dv);
  return p.causal ? bwd_kv<128, true>(p, q, k, v, dO, lse, delta, dk, dv)
                  : bwd_kv<128, false>(p, q, k, v, dO, lse, delta, dk, dv);
}

hipError_t launch_bwd_dq_f32(const Problem& p, const float* q, const float* k, const float* v, const float* dO,
                             const float* lse, float* dq, const void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, false);
  const float* delta = (const float*)((const char*)workspace + ws.delta_off);
  if (p.d == 64)
    return p.causal ? bwd_q<64, true>(p, q, k, v, dO, lse, delta, dq) : bwd_q<64, false>(p, q, k, v, dO, lse, delta, dq);
  return p.causal ? bwd_q<128, true>(p, q, k, v, dO, lse, delta, dq) : bwd_q<128, false>(p, q, k, v, dO, lse, delta, dq);
}

}  // namespace fa
