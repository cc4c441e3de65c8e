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
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, float* __restrict__ O,
                                                     float* __restrict__ LSE, int H, int N, float scale,
                                                     const int32_t* __restrict__ seqlens,
                                                     const uint8_t* __restrict__ bmask, Dropout dr) {
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
    // dropout: keep words of this query for the tile's 32 keys (halves h = 0, 1)
    u32x4 kw[2] = {};
    if constexpr (DROP) {
      kw[0] = dropout_words(dr, (uint32_t)(b * H + h), query, k0 / 32, 0);
      kw[1] = dropout_words(dr, (uint32_t)(b * H + h), query, k0 / 32, 1);
    }
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
      float p = expf(s[j] - m_use);
      l += p;
      if constexpr (DROP) p = dropout_keep(dr, kw[(j >> 2) & 1][j >> 3], j & 3) ? p : 0.f;  // scaled at the end
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vs[j][c], acc[c]);
    }
    m = m_new;
  }
  if (query < N) {
    const bool has = l > 0.f;
    const float inv = has ? (DROP ? dr.scale : 1.f) / l : 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) O[(row0 + query) * D + c] = acc[c] * inv;
    LSE[row0 + query] = has ? m + logf(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------------
// Backward, dK and dV: thread = key row (its K and V rows staged in LDS), loop over query tiles.
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(64) void bwd_kv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V, const float* __restrict__ dO,
                                                        const float* __restrict__ LSE, const float* __restrict__ DELTA,
                                                        float* __restrict__ dK, float* __restrict__ dV, int H, int N,
                                                        float scale, const int32_t* __restrict__ seqlens,
                                                        const uint8_t* __restrict__ bmask, Dropout dr) {
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
      del_s[threadIdx.x] = -DELTA[row0 + qq];  // (the workspace holds -D)
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
      float pz = p;  // dropout: the kept probability (scaled) feeds dV, the kept dP (scaled) feeds dS
      if constexpr (DROP) {
        const u32x4 w = dropout_words(dr, (uint32_t)(b * H + h), query, key / 32, (key >> 2) & 1);
        const bool keep = dropout_keep(dr, w[(key & 31) >> 3], key & 3);
        pz = keep ? p * dr.scale : 0.f;
        dp = keep ? dp * dr.scale : 0.f;
      }
      const float dsv = p * (dp - del_s[i]);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        dv[c] = fmaf(pz, gs[i][c], dv[c]);
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
template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(64) void bwd_q_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       const float* __restrict__ LSE, const float* __restrict__ DELTA,
                                                       float* __restrict__ dQ, int H, int N, float scale,
                                                       const int32_t* __restrict__ seqlens,
                                                       const uint8_t* __restrict__ bmask, Dropout dr) {
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
  const float del = -DELTA[row0 + qrow];  // (the workspace holds -D)
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
    u32x4 kw[2] = {};
    if constexpr (DROP) {
      kw[0] = dropout_words(dr, (uint32_t)(b * H + h), query, k0 / 32, 0);
      kw[1] = dropout_words(dr, (uint32_t)(b * H + h), query, k0 / 32, 1);
    }
    for (int j = 0; j < kF32Tile; ++j) {
      if (!visible<CAUSAL>(query, k0 + j, L)) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = fmaf(qr[threadIdx.x][c], ks[j][c], s);
        dp = fmaf(gr[threadIdx.x][c], vs[j][c], dp);
      }
      const float p = expf(s * scale - lse);
      if constexpr (DROP) dp = dropout_keep(dr, kw[(j >> 2) & 1][j >> 3], j & 3) ? dp * dr.scale : 0.f;
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

Dropout dropout_of(const Problem& p) {
  return Dropout{p.drop_k0, p.drop_k1, p.drop_off2, p.drop_t, 256.f / (float)p.drop_t};
}

template <int D, bool CAUSAL, bool DROP>
hipError_t fwd(const Problem& p, const float* q, const float* k, const float* v, float* o, float* lse) {
  dim3 grid((p.N + kF32Rows - 1) / kF32Rows, p.H, p.B);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, DROP>), grid, dim3(64), 0, p.stream, q, k, v, o, lse, p.H, p.N, p.scale,
                     p.seqlens, p.block_mask, dropout_of(p));
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool DROP>
hipError_t bwd_kv(const Problem& p, const float* q, const float* k, const float* v, const float* dO, const float* lse,
                  const float* delta, float* dk, float* dv) {
  dim3 grid((p.N + kF32Rows - 1) / kF32Rows, p.H, p.B);
  hipLaunchKernelGGL((bwd_kv_f32_kernel<D, CAUSAL, DROP>), grid, dim3(64), 0, p.stream, q, k, v, dO, lse, delta, dk,
                     dv, p.H, p.N, p.scale, p.seqlens, p.block_mask, dropout_of(p));
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool DROP>
hipError_t bwd_q(const Problem& p, const float* q, const float* k, const float* v, const float* dO, const float* lse,
                 const float* delta, float* dq) {
  dim3 grid((p.N + kF32Rows - 1) / kF32Rows, p.H, p.B);
  hipLaunchKernelGGL((bwd_q_f32_kernel<D, CAUSAL, DROP>), grid, dim3(64), 0, p.stream, q, k, v, dO, lse, delta, dq,
                     p.H, p.N, p.scale, p.seqlens, p.block_mask, dropout_of(p));
  return hipGetLastError();
}

// Keep mask as bytes: one thread per (bh, query, 32-key block), both halves.
__global__ __launch_bounds__(256) void dropout_mask_kernel(uint8_t* __restrict__ keep, int N, int64_t total,
                                                           Dropout dr) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int nb32 = (N + 31) / 32;
  const int jb = (int)(idx % nb32);
  const int64_t rest = idx / nb32;
  const int i = (int)(rest % N);
  const int64_t bh = rest / N;
  uint8_t* row = keep + (bh * N + i) * (int64_t)N;
  for (int h = 0; h < 2; ++h) {
    const u32x4 w = dropout_words(dr, (uint32_t)bh, i, jb, h);
    for (int g = 0; g < 4; ++g)
      for (int e = 0; e < 4; ++e) {
        const int j = 32 * jb + 8 * g + 4 * h + e;
        if (j < N) row[j] = dropout_keep(dr, w[g], e) ? 1 : 0;
      }
  }
}

template <int D, bool DROP>
hipError_t fwd_c(const Problem& p, const float* q, const float* k, const float* v, float* o, float* lse) {
  return p.causal ? fwd<D, true, DROP>(p, q, k, v, o, lse) : fwd<D, false, DROP>(p, q, k, v, o, lse);
}
template <int D, bool DROP>
hipError_t bwd_kv_c(const Problem& p, const float* q, const float* k, const float* v, const float* dO, const float* lse,
                    const float* delta, float* dk, float* dv) {
  return p.causal ? bwd_kv<D, true, DROP>(p, q, k, v, dO, lse, delta, dk, dv)
                  : bwd_kv<D, false, DROP>(p, q, k, v, dO, lse, delta, dk, dv);
}
template <int D, bool DROP>
hipError_t bwd_q_c(const Problem& p, const float* q, const float* k, const float* v, const float* dO, const float* lse,
                   const float* delta, float* dq) {
  return p.causal ? bwd_q<D, true, DROP>(p, q, k, v, dO, lse, delta, dq)
                  : bwd_q<D, false, DROP>(p, q, k, v, dO, lse, delta, dq);
}

}  // namespace

hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o, float* lse) {
  if (p.d == 64) return p.dropout ? fwd_c<64, true>(p, q, k, v, o, lse) : fwd_c<64, false>(p, q, k, v, o, lse);
  return p.dropout ? fwd_c<128, true>(p, q, k, v, o, lse) : fwd_c<128, false>(p, q, k, v, o, lse);
}

hipError_t launch_bwd_dkdv_f32(const Problem& p, const float* q, const float* k, const float* v, const float* dO,
                               const float* lse, float* dk, float* dv, const void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, false);
  const float* delta = (const float*)((const char*)workspace + ws.delta_off);
  if (p.d == 64)
    return p.dropout ? bwd_kv_c<64, true>(p, q, k, v, dO, lse, delta, dk, dv)
                     : bwd_kv_c<64, false>(p, q, k, v, dO, lse, delta, dk, dv);
  return p.dropout ? bwd_kv_c<128, true>(p, q, k, v, dO, lse, delta, dk, dv)
                   : bwd_kv_c<128, false>(p, q, k, v, dO, lse, delta, dk, dv);
}

hipError_t launch_bwd_dq_f32(const Problem& p, const float* q, const float* k, const float* v, const float* dO,
                             const float* lse, float* dq, const void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, false);
  const float* delta = (const float*)((const char*)workspace + ws.delta_off);
  if (p.d == 64)
    return p.dropout ? bwd_q_c<64, true>(p, q, k, v, dO, lse, delta, dq) : bwd_q_c<64, false>(p, q, k, v, dO, lse, delta, dq);
  return p.dropout ? bwd_q_c<128, true>(p, q, k, v, dO, lse, delta, dq) : bwd_q_c<128, false>(p, q, k, v, dO, lse, delta, dq);
}

hipError_t launch_dropout_mask(const Problem& p, uint8_t* keep) {
  const int64_t total = (int64_t)p.B * p.H * p.N * ((p.N + 31) / 32);
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, p.stream, keep, p.N,
                     total, dropout_of(p));
  return hipGetLastError();
}

}  // namespace fa
