// Backward of exact attention, bf16 inputs, fp32 accumulation, on gfx950 matrix cores.
//
// The backward never reads a stored N x N matrix: it recomputes each block of probabilities from
// Q, K and the per-row log-sum-exp the forward kept (NOTE-005: FlashAttention, "Method" and "Key
// components"; aicassindra FlashAttention architecture page, "The architecture: every piece
// explained").  The gradient formulas are the chain rule through softmax for the loss sum(dO*O):
//   P = exp(S - LSE),  dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D),  dK = scale dS^T Q,  dQ = scale dS K.
//
// Three kernels:
//   bwd_pre      D_i = sum_c dO_ic O_ic (fp32) and zero the fp32 dQ accumulator;
//   bwd_main     one workgroup per 128 keys of a (batch, head), 4 waves x 32 keys.  K and V of the
//                wave stay in registers; dK^T and dV^T accumulate in registers for the whole
//                walk over query tiles (64 rows each, double-buffered in LDS with direct
//                global->LDS loads).  Per tile: S = Q K^T and dP = dO V^T on MFMA, P and dS on
//                the VALU, dV^T += dO^T P and dK^T += Q^T dS on MFMA with dO^T / Q^T read through
//                the transposing LDS read.  dS^T of the four waves meets in LDS, and the
//                workgroup adds dS K for all its 128 keys to the fp32 dQ accumulator with one
//                set of float atomics (four times fewer atomics than per-wave partial sums);
//   bwd_convert  dq = bf16(scale * dQ accumulator).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdKeysPerWave = 32;
constexpr int kBwdBc = kBwdWaves * kBwdKeysPerWave;  // 128 keys per workgroup
constexpr int kBwdBr = 64;                           // query rows per tile

// ---------------------------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic; zero the dQ accumulator row.  D/8 threads per row, 8 elements each.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      float* __restrict__ delta, float* __restrict__ dqacc,
                                                      int64_t rows) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float sum = 0.f;
  if (row < rows) {
    const T* o = O + row * D + part * 8;
    const T* g = dO + row * D + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += (float)o[e] * (float)g[e];
    if (dqacc != nullptr) {
      float4* z = (float4*)(dqacc + row * D + part * 8);
      z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, TPR);
  if (row < rows && part == 0) delta[row] = sum;
}

// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_convert_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
                                                          float scale, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = ((const float4*)acc)[2 * i];
  const float4 b = ((const float4*)acc)[2 * i + 1];
  const bf16x4 lo = pack4(a.x * scale, a.y * scale, a.z * scale, a.w * scale);
  const bf16x4 hi = pack4(b.x * scale, b.y * scale, b.z * scale, b.w * scale);
  ((bf16x8*)dq)[i] = cat(lo, hi);
}

// ---------------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                          const float* __restrict__ LSE,
                                                          const float* __restrict__ DELTA, float* __restrict__ dQacc,
                                                          __bf16* __restrict__ dK, __bf16* __restrict__ dV, int H,
                                                          int N, float scale, float c_log2,
                                                          const int32_t* __restrict__ seqlens) {
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int QTILE = kBwdBr * D * 2;      // bytes of a Q or dO tile
  constexpr int LOADS = kBwdBr * CH / 256;   // 16-byte loads per thread per tile and tensor
  constexpr int DS = D / 16;                 // k-steps over d
  constexpr int DT = D / 32;                 // 32-wide d tiles
  constexpr int BUF = 2 * QTILE + 2 * kBwdBr * 4;  // Q | dO | LSE | DELTA
  constexpr int DQ_TILES = (2 * DT) / kBwdWaves;   // 32x32 dQ tiles per wave (2 for d=128, 1 for d=64)
  static_assert(2 * QTILE >= kBwdBc * D * 2, "K staging must fit in one buffer");
  __shared__ __attribute__((aligned(1024))) char buf0_raw[BUF];
  __shared__ __attribute__((aligned(1024))) char buf1_raw[BUF];
  __shared__ __attribute__((aligned(1024))) char dst_raw[kBwdBc * kBwdBr * 2];  // dS^T [128 keys][64 q]
  FA_LDS char* buf0 = (FA_LDS char*)buf0_raw;
  FA_LDS char* buf1 = (FA_LDS char*)buf1_raw;
  FA_LDS char* dsT = (FA_LDS char*)dst_raw;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t row0 = ((int64_t)b * H + h) * N;
  const __bf16* Qh = Q + row0 * D;
  const __bf16* Kh = K + row0 * D;
  const __bf16* Vh = V + row0 * D;
  const __bf16* dOh = dO + row0 * D;
  const float* LSEh = LSE + row0;
  const float* DELh = DELTA + row0;
  float* dQh = dQacc + row0 * D;

  const int L = PADDED ? clamp_len(seqlens, b, N) : N;
  const int k0 = blockIdx.x * kBwdBc;
  const int kw = k0 + wave * kBwdKeysPerWave;
  const int my_key = kw + l32;

  f32x16 dvt[DT], dkt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dvt[dt] = zero16();
    dkt[dt] = zero16();
  }

  if (k0 < L) {
    // ---- stationary operands: K and V (B operands of S = Q K^T and dP = dO V^T)
    bf16x8 kb[DS], vb[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      if (my_key < N) {
        kb[ds] = *(const bf16x8*)(Kh + (int64_t)my_key * D + 16 * ds + 8 * half);
        vb[ds] = *(const bf16x8*)(Vh + (int64_t)my_key * D + 16 * ds + 8 * half);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kb[ds][e] = (__bf16)0.f;
          vb[ds][e] = (__bf16)0.f;
        }
      }
    }
    // ---- K of all 128 keys as the B operand of dQ = dS K for this wave's d tile: lane holds
    // d = 32 dtq + l32 and, for k-step ks, keys 16 ks + 4 half + 0..3, 16 ks + 8 + 4 half + 0..3.
    // Stage the [128][D] K block in buf1 and read it transposed.
    const int dtq = (DT == 4) ? wave : (wave & 1);
    bf16x8 kq[kBwdBc / 16];
    {
      for (int p = threadIdx.x; p < kBwdBc * CH; p += 256) {
        const int r = p / CH, c = p % CH;
        const int key = min(k0 + r, N - 1);
        *(FA_LDS u32x4*)(buf1 + tile_off<D>(r, 8 * c)) = *(const u32x4*)(Kh + (int64_t)key * D + 8 * c);
      }
      __syncthreads();
      const int dcol = 32 * dtq + 16 * (g16 & 1) + 4 * (j16 & 3);
#pragma unroll
      for (int ks = 0; ks < kBwdBc / 16; ++ks) {
        const int krow = 16 * ks + 4 * (g16 >> 1) + (j16 >> 2);
        kq[ks] = cat(lds_read_tr(buf1, tile_off<D>(krow, dcol)), lds_read_tr(buf1, tile_off<D>(krow + 8, dcol)));
      }
      __syncthreads();
    }

    const int nqt = (N + kBwdBr - 1) / kBwdBr;
    const int it0 = CAUSAL ? (k0 / kBwdBr) : 0;

    auto issue_tile = [&](int it, FA_LDS char* dst) {
      const int qbase = it * kBwdBr;
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int slot = (n * kBwdWaves + wave) * 64;
        const int p = slot + lane;
        const int r = p / CH;
        const int c = (p % CH) ^ swz(r);
        const int q = min(qbase + r, N - 1);
        gload_lds16(Qh + (int64_t)q * D + 8 * c, dst + slot * 16);
        gload_lds16(dOh + (int64_t)q * D + 8 * c, dst + QTILE + slot * 16);
      }
      if (wave < 2) {
        const int q = min(qbase + lane, N - 1);
        gload_lds4(wave == 0 ? (const void*)(LSEh + q) : (const void*)(DELh + q), dst + 2 * QTILE + wave * kBwdBr * 4);
      }
    };

    auto step = [&](int it, const FA_LDS char* cur, FA_LDS char* nxt) {
      wait_vmem();
      __syncthreads();
      if (it + 1 < nqt) issue_tile(it + 1, nxt);
      const FA_LDS char* qs_t = cur;
      const FA_LDS char* do_t = cur + QTILE;
      const FA_LDS float* lse_t = (const FA_LDS float*)(cur + 2 * QTILE);
      const FA_LDS float* del_t = lse_t + kBwdBr;
      const int qi0 = it * kBwdBr;
      // wave-uniform: does any (query, key) pair of this wave's block survive the mask?
      const bool active = (kw < L) && (!CAUSAL || kw <= qi0 + kBwdBr - 1);
      if (active) {
        f32x16 s[2], dp[2];
        s[0] = zero16(); s[1] = zero16(); dp[0] = zero16(); dp[1] = zero16();
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) {
            const uint32_t off = tile_off<D>(32 * qs + l32, 16 * ds + 8 * half);
            const bf16x8 qa = lds_read_b128(qs_t, off);
            const bf16x8 da = lds_read_b128(do_t, off);
            s[qs] = mfma32x32x16(qa, kb[ds], s[qs]);
            dp[qs] = mfma32x32x16(da, vb[ds], dp[qs]);
          }
        }
        // ---- P and dS (fp32), masked; lane holds key my_key, queries 8 g + 4 half + 0..3
        const bool edge = (kw + kBwdKeysPerWave > L) || (qi0 + kBwdBr > N) || (CAUSAL && kw + 31 > qi0);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int qloc = 32 * qs + 8 * gq + 4 * half;
            const f32x4 lse4 = *(const FA_LDS f32x4*)(lse_t + qloc);
            const f32x4 del4 = *(const FA_LDS f32x4*)(del_t + qloc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * gq + e;
              float p = fast_exp2(fmaf(s[qs][r], c_log2, -lse4[e] * kLog2e));
              if (edge) {
                const int query = qi0 + qloc + e;
                const bool vis = my_key < L && query < N && (!CAUSAL || my_key <= query);
                p = vis ? p : 0.f;
              }
              s[qs][r] = p;
              dp[qs][r] = p * (dp[qs][r] - del4[e]);
            }
          }
        }
        bf16x8 pb[4], db[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          pb[ks] = pack8(s[ks >> 1], 8 * (ks & 1));
          db[ks] = pack8(dp[ks >> 1], 8 * (ks & 1));
        }
        // ---- dV^T += dO^T P ; dK^T += Q^T dS  (A operands through the transposing read)
        const int trow = 4 * (g16 >> 1) + (j16 >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int dcol = 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3);
          const uint32_t dbase = lds_addr(do_t) + tile_off<D>(trow, dcol);
          const uint32_t qbase = lds_addr(qs_t) + tile_off<D>(trow, dcol);
          u32x2 a0 = lds_read_tr_asm<0 * D * 2>(dbase), a1 = lds_read_tr_asm<8 * D * 2>(dbase);
          u32x2 a2 = lds_read_tr_asm<16 * D * 2>(dbase), a3 = lds_read_tr_asm<24 * D * 2>(dbase);
          u32x2 a4 = lds_read_tr_asm<32 * D * 2>(dbase), a5 = lds_read_tr_asm<40 * D * 2>(dbase);
          u32x2 a6 = lds_read_tr_asm<48 * D * 2>(dbase), a7 = lds_read_tr_asm<56 * D * 2>(dbase);
          u32x2 b0 = lds_read_tr_asm<0 * D * 2>(qbase), b1 = lds_read_tr_asm<8 * D * 2>(qbase);
          u32x2 b2 = lds_read_tr_asm<16 * D * 2>(qbase), b3 = lds_read_tr_asm<24 * D * 2>(qbase);
          u32x2 b4 = lds_read_tr_asm<32 * D * 2>(qbase), b5 = lds_read_tr_asm<40 * D * 2>(qbase);
          u32x2 b6 = lds_read_tr_asm<48 * D * 2>(qbase), b7 = lds_read_tr_asm<56 * D * 2>(qbase);
          lds_wait(a0, a1, a2, a3, a4, a5, a6, a7);
          lds_wait(b0, b1, b2, b3, b4, b5, b6, b7);
          dvt[dt] = mfma32x32x16(cat(a0, a1), pb[0], dvt[dt]);
          dvt[dt] = mfma32x32x16(cat(a2, a3), pb[1], dvt[dt]);
          dvt[dt] = mfma32x32x16(cat(a4, a5), pb[2], dvt[dt]);
          dvt[dt] = mfma32x32x16(cat(a6, a7), pb[3], dvt[dt]);
          dkt[dt] = mfma32x32x16(cat(b0, b1), db[0], dkt[dt]);
          dkt[dt] = mfma32x32x16(cat(b2, b3), db[1], dkt[dt]);
          dkt[dt] = mfma32x32x16(cat(b4, b5), db[2], dkt[dt]);
          dkt[dt] = mfma32x32x16(cat(b6, b7), db[3], dkt[dt]);
        }
        // ---- dS^T -> LDS [key][q] (bf16): lane writes key 32 wave + l32, 4 queries per store
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int qloc = 32 * qs + 8 * gq + 4 * half;
            *(FA_LDS bf16x4*)(dsT + tile_off<kBwdBr>(32 * wave + l32, qloc)) =
                pack4(dp[qs][4 * gq], dp[qs][4 * gq + 1], dp[qs][4 * gq + 2], dp[qs][4 * gq + 3]);
          }
      } else {
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int qloc = 32 * qs + 8 * gq + 4 * half;
            *(FA_LDS bf16x4*)(dsT + tile_off<kBwdBr>(32 * wave + l32, qloc)) = pack4(0.f, 0.f, 0.f, 0.f);
          }
      }
      __syncthreads();
      // ---- dQ[q][d] += dS[q][key] K[key][d] over the 128 keys, then fp32 atomics (unscaled)
#pragma unroll
      for (int tq = 0; tq < DQ_TILES; ++tq) {
        const int qs = (DT == 4) ? tq : (wave >> 1);
        f32x16 accq = zero16();
        const uint32_t sbase = lds_addr(dsT) + tile_off<kBwdBr>(4 * (g16 >> 1) + (j16 >> 2),
                                                              32 * qs + 16 * (g16 & 1) + 4 * (j16 & 3));
        u32x2 t0 = lds_read_tr_asm<0 * kBwdBr * 2>(sbase), t1 = lds_read_tr_asm<8 * kBwdBr * 2>(sbase);
        u32x2 t2 = lds_read_tr_asm<16 * kBwdBr * 2>(sbase), t3 = lds_read_tr_asm<24 * kBwdBr * 2>(sbase);
        u32x2 t4 = lds_read_tr_asm<32 * kBwdBr * 2>(sbase), t5 = lds_read_tr_asm<40 * kBwdBr * 2>(sbase);
        u32x2 t6 = lds_read_tr_asm<48 * kBwdBr * 2>(sbase), t7 = lds_read_tr_asm<56 * kBwdBr * 2>(sbase);
        u32x2 t8 = lds_read_tr_asm<64 * kBwdBr * 2>(sbase), t9 = lds_read_tr_asm<72 * kBwdBr * 2>(sbase);
        u32x2 t10 = lds_read_tr_asm<80 * kBwdBr * 2>(sbase), t11 = lds_read_tr_asm<88 * kBwdBr * 2>(sbase);
        u32x2 t12 = lds_read_tr_asm<96 * kBwdBr * 2>(sbase), t13 = lds_read_tr_asm<104 * kBwdBr * 2>(sbase);
        u32x2 t14 = lds_read_tr_asm<112 * kBwdBr * 2>(sbase), t15 = lds_read_tr_asm<120 * kBwdBr * 2>(sbase);
        lds_wait(t0, t1, t2, t3, t4, t5, t6, t7);
        lds_wait(t8, t9, t10, t11, t12, t13, t14, t15);
        accq = mfma32x32x16(cat(t0, t1), kq[0], accq);
        accq = mfma32x32x16(cat(t2, t3), kq[1], accq);
        accq = mfma32x32x16(cat(t4, t5), kq[2], accq);
        accq = mfma32x32x16(cat(t6, t7), kq[3], accq);
        accq = mfma32x32x16(cat(t8, t9), kq[4], accq);
        accq = mfma32x32x16(cat(t10, t11), kq[5], accq);
        accq = mfma32x32x16(cat(t12, t13), kq[6], accq);
        accq = mfma32x32x16(cat(t14, t15), kq[7], accq);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int query = qi0 + 32 * qs + 8 * (r >> 2) + 4 * half + (r & 3);
          if (query < N) unsafeAtomicAdd(dQh + (int64_t)query * D + 32 * dtq + l32, accq[r]);
        }
      }
    };

    if (it0 < nqt) issue_tile(it0, buf0);
    for (int it = it0; it < nqt; it += 2) {
      step(it, buf0, buf1);
      if (it + 1 < nqt) step(it + 1, buf1, buf0);
    }
  }

  // ---- dK = scale dS^T Q, dV: lane holds key my_key, d = 32 dt + 8 g + 4 half + 0..3
  if (my_key < N) {
    __bf16* dkrow = dK + (row0 + my_key) * D;
    __bf16* dvrow = dV + (row0 + my_key) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dt + 8 * gq + 4 * half;
        *(bf16x4*)(dkrow + d0) = pack4(dkt[dt][4 * gq] * scale, dkt[dt][4 * gq + 1] * scale,
                                       dkt[dt][4 * gq + 2] * scale, dkt[dt][4 * gq + 3] * scale);
        *(bf16x4*)(dvrow + d0) = pack4(dvt[dt][4 * gq], dvt[dt][4 * gq + 1], dvt[dt][4 * gq + 2], dvt[dt][4 * gq + 3]);
      }
  }
}

template <int D, bool CAUSAL, bool PADDED>
hipError_t launch_main(const Problem& p, const void* q, const void* k, const void* v, const void* dO, const float* lse,
                       const float* delta, float* dqacc, void* dk, void* dv) {
  dim3 grid((p.N + kBwdBc - 1) / kBwdBc, p.H, p.B);
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, PADDED>), grid, dim3(256), 0, p.stream, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, lse, delta, dqacc, (__bf16*)dk,
                     (__bf16*)dv, p.H, p.N, p.scale, p.scale * kLog2e, p.seqlens);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_pre(const Problem& p, const void* o, const void* dO, float* delta, float* dqacc) {
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  constexpr int rows_per_block = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D, T>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(256), 0, p.stream, (const T*)o, (const T*)dO, delta, dqacc, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prepare(const Problem& p, bool bf16, const void* o, const void* dO, void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, bf16);
  float* delta = (float*)((char*)workspace + ws.delta_off);
  if (bf16) {
    float* dqacc = (float*)((char*)workspace + ws.dqacc_off);
    return p.d == 64 ? launch_pre<64, __bf16>(p, o, dO, delta, dqacc) : launch_pre<128, __bf16>(p, o, dO, delta, dqacc);
  }
  return p.d == 64 ? launch_pre<64, float>(p, o, dO, delta, nullptr) : launch_pre<128, float>(p, o, dO, delta, nullptr);
}

hipError_t launch_bwd_main_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                                const float* lse, void* dk, void* dv, void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, true);
  const float* delta = (const float*)((char*)workspace + ws.delta_off);
  float* dqacc = (float*)((char*)workspace + ws.dqacc_off);
  const bool pad = p.seqlens != nullptr;
  if (p.d == 64) {
    if (p.causal)
      return pad ? launch_main<64, true, true>(p, q, k, v, dO, lse, delta, dqacc, dk, dv)
                 : launch_main<64, true, false>(p, q, k, v, dO, lse, delta, dqacc, dk, dv);
    return pad ? launch_main<64, false, true>(p, q, k, v, dO, lse, delta, dqacc, dk, dv)
               : launch_main<64, false, false>(p, q, k, v, dO, lse, delta, dqacc, dk, dv);
  }
  if (p.causal)
    return pad ? launch_main<128, true, true>(p, q, k, v, dO, lse, delta, dqacc, dk, dv)
               : launch_main<128, true, false>(p, q, k, v, dO, lse, delta, dqacc, dk, dv);
  return pad ? launch_main<128, false, true>(p, q, k, v, dO, lse, delta, dqacc, dk, dv)
             : launch_main<128, false, false>(p, q, k, v, dO, lse, delta, dqacc, dk, dv);
}

hipError_t launch_bwd_finish_bf16(const Problem& p, void* dq, void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, true);
  const float* dqacc = (const float*)((char*)workspace + ws.dqacc_off);
  const int64_t n8 = (int64_t)p.B * p.H * p.N * p.d / 8;
  if (p.d == 64)
    hipLaunchKernelGGL((bwd_convert_kernel<64>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, p.stream, dqacc,
                       (__bf16*)dq, p.scale, n8);
  else
    hipLaunchKernelGGL((bwd_convert_kernel<128>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, p.stream, dqacc,
                       (__bf16*)dq, p.scale, n8);
  return hipGetLastError();
}

}  // namespace fa
