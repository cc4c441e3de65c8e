// The pages' own schedule of exact attention, instrumented for its HBM traffic (the IO-complexity
// measurement; not a throughput path).
//
// NOTE-005: FlashAttention, "Method": with SRAM of M elements set B_c = ceil(M / 4d) and
// B_r = min(ceil(M / 4d), d); loop over the K, V blocks in the outer loop and over the Q blocks in
// the inner one; load the tiles into SRAM, compute the block of Q K^T there and update the output
// with the online softmax, keeping the running maximum m and normaliser l -- here, as in that
// algorithm, O, m and l live in HBM between blocks and are read and written back for every
// (K/V block, Q block) pair.  "Key results", Theorem 2: for d <= M <= N d this schedule makes
// Theta(N^2 d^2 / M) HBM accesses.  The budget M is set by the caller (the LDS is limited
// artificially to sweep it); the tiles are held in LDS as fp32, so M counts 4-byte elements.
//
// One workgroup per (batch, head) walks every (j, i) pair in order (the algorithm's loops, no
// parallelism inside a head, so the access pattern is exactly the algorithm's).  256 threads share
// the products; fp32 FMAs on the vector ALUs.
#include "fa.h"
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kKvoThreads = 256;

template <int D>
__global__ __launch_bounds__(kKvoThreads) void fwd_kv_outer_kernel(const __bf16* __restrict__ Q,
                                                                    const __bf16* __restrict__ K,
                                                                    const __bf16* __restrict__ V,
                                                                    __bf16* __restrict__ O, float* __restrict__ LSE,
                                                                    float* __restrict__ Ow, float* __restrict__ Mw,
                                                                    float* __restrict__ Lw, int N, float scale,
                                                                    int Bc, int Br) {
  extern __shared__ float smem[];
  float* ks = smem;               // [Bc][D]
  float* vs = ks + Bc * D;        // [Bc][D]
  float* qs = vs + Bc * D;        // [Br][D]
  float* os = qs + Br * D;        // [Br][D]
  float* ss = os + Br * D;        // [Br][Bc]: S, then P~
  float* fa_ = ss + Br * Bc;      // [Br]: e^(m - m_new) l / l_new
  float* fb_ = fa_ + Br;          // [Br]: e^(m~ - m_new) / l_new
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * N;
  const __bf16* Qh = Q + row0 * D;
  const __bf16* Kh = K + row0 * D;
  const __bf16* Vh = V + row0 * D;
  float* Oh = Ow + row0 * D;
  float* Mh = Mw + row0;
  float* Lh = Lw + row0;
  const int Tc = (N + Bc - 1) / Bc, Tr = (N + Br - 1) / Br;

  // O = 0, l = 0, m = -inf in HBM
  for (int64_t x = tid; x < (int64_t)N * D; x += kKvoThreads) Oh[x] = 0.f;
  for (int x = tid; x < N; x += kKvoThreads) {
    Mh[x] = -INFINITY;
    Lh[x] = 0.f;
  }
  __threadfence_block();
  __syncthreads();

  for (int j = 0; j < Tc; ++j) {
    const int k0 = j * Bc, nk = min(Bc, N - k0);
    // load K_j, V_j (rows past N are never used)
    for (int x = tid; x < nk * D; x += kKvoThreads) {
      ks[x] = (float)Kh[(int64_t)k0 * D + x];
      vs[x] = (float)Vh[(int64_t)k0 * D + x];
    }
    for (int i = 0; i < Tr; ++i) {
      const int q0 = i * Br, nq = min(Br, N - q0);
      // load Q_i, O_i
      for (int x = tid; x < nq * D; x += kKvoThreads) {
        qs[x] = (float)Qh[(int64_t)q0 * D + x];
        os[x] = Oh[(int64_t)q0 * D + x];
      }
      __syncthreads();
      // S_ij = scale Q_i K_j^T
      for (int x = tid; x < nq * Bc; x += kKvoThreads) {
        const int r = x / Bc, c = x % Bc;
        float acc = 0.f;
        if (c < nk) {
#pragma unroll 8
          for (int e = 0; e < D; ++e) acc = fmaf(qs[r * D + e], ks[c * D + e], acc);
        }
        ss[x] = c < nk ? acc * scale : -INFINITY;
      }
      __syncthreads();
      // row statistics: m~ = rowmax S, P~ = exp(S - m~), l~ = rowsum P~; new m and l
      for (int r = tid; r < nq; r += kKvoThreads) {
        float mt = -INFINITY;
        for (int c = 0; c < nk; ++c) mt = fmaxf(mt, ss[r * Bc + c]);
        float lt = 0.f;
        for (int c = 0; c < Bc; ++c) {
          const float p = c < nk ? expf(ss[r * Bc + c] - mt) : 0.f;
          ss[r * Bc + c] = p;
          lt += p;
        }
        const float m_old = Mh[q0 + r], l_old = Lh[q0 + r];
        const float m_new = fmaxf(m_old, mt);
        const float ea = expf(m_old - m_new), eb = expf(mt - m_new);
        const float l_new = ea * l_old + eb * lt;
        fa_[r] = ea * l_old / l_new;
        fb_[r] = eb / l_new;
        Mh[q0 + r] = m_new;
        Lh[q0 + r] = l_new;
        if (j == Tc - 1) LSE[row0 + q0 + r] = m_new + logf(l_new);
      }
      __syncthreads();
      // O_i = diag(l_new)^-1 (diag(l) e^(m - m_new) O_i + e^(m~ - m_new) P~ V_j), written back
      for (int x = tid; x < nq * D; x += kKvoThreads) {
        const int r = x / D, c = x % D;
        float pv = 0.f;
        for (int e = 0; e < nk; ++e) pv = fmaf(ss[r * Bc + e], vs[e * D + c], pv);
        const float o = fa_[r] * os[x] + fb_[r] * pv;
        if (j == Tc - 1) O[(row0 + q0) * D + x] = (__bf16)o;
        else Oh[(int64_t)q0 * D + x] = o;
      }
      __syncthreads();
    }
  }
}

}  // namespace

KvOuterTiles kv_outer_tiles(int d, size_t lds_bytes) {
  KvOuterTiles t{};
  const int64_t m = (int64_t)(lds_bytes / 4);  // fp32 elements
  t.Bc = (int)((m + 4 * d - 1) / (4 * d));
  t.Br = t.Bc < d ? t.Bc : d;
  t.smem = ((size_t)2 * t.Bc * d + (size_t)2 * t.Br * d + (size_t)t.Br * t.Bc + 2 * (size_t)t.Br) * 4;
  return t;
}

hipError_t launch_fwd_kv_outer(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse,
                               void* workspace, size_t lds_bytes) {
  const KvOuterTiles t = kv_outer_tiles(p.d, lds_bytes);
  const size_t rows = (size_t)p.B * p.H * p.N;
  float* Ow = (float*)workspace;
  float* Mw = Ow + rows * p.d;
  float* Lw = Mw + rows;
  const unsigned grid = (unsigned)(p.B * p.H);
  if (p.d == 64) {
    hipFuncSetAttribute((const void*)fwd_kv_outer_kernel<64>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)t.smem);
    hipLaunchKernelGGL(fwd_kv_outer_kernel<64>, dim3(grid), dim3(kKvoThreads), t.smem, p.stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, Ow, Mw, Lw, p.N, p.scale, t.Bc, t.Br);
  } else {
    hipFuncSetAttribute((const void*)fwd_kv_outer_kernel<128>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)t.smem);
    hipLaunchKernelGGL(fwd_kv_outer_kernel<128>, dim3(grid), dim3(kKvoThreads), t.smem, p.stream, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, Ow, Mw, Lw, p.N, p.scale, t.Bc, t.Br);
  }
  return hipGetLastError();
}

}  // namespace fa
