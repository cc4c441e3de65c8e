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
//   bwd_pre      D_i = sum_c dO_ic O_ic and LSE_i log2(e) (fp32), and zero the fp32 dQ accumulator;
//   bwd_main     one workgroup per 128 keys of a (batch, head): 4 waves x 32 keys, one wave per
//                SIMD.  K and V of the wave stay in registers (B operands of S = Q K^T and
//                dP = dO V^T), and dK^T, dV^T accumulate in registers over the whole walk of
//                64-row query tiles.  The query tiles (Q, dO, LSE log2 e, D) stream through a
//                three-stage LDS ring filled by direct global->LDS loads two tiles ahead.  Per
//                tile u, one barrier, then
//                  A: dQ(u-1) = dS(u-1) K on the matrix cores (dS^T of all four waves from LDS),
//                     interleaved with P(u) = exp2(S scale log2 e - LSE log2 e) and
//                     dS(u) = P (dP - D) on the VALU; dS^T(u) goes to LDS.  dQ(u-1) is added to
//                     the fp32 accumulator with float atomics (one per element per key block) at
//                     the start of the next iteration, next to the tile loads, so the wait for
//                     those loads never waits for freshly issued atomics;
//                  B: dV^T += dO^T P(u), dK^T += Q^T dS(u) (dO^T, Q^T via transposing LDS reads);
//                  C: S(u+1) = Q K^T, dP(u+1) = dO V^T.
//                Tiles with hidden pairs (causal diagonal, key padding, ragged tail) first set the
//                hidden scores to -inf (so P = 0 and dS = 0 there).  The accumulator has its rows
//                padded to a multiple of 64, so tail tiles need no branches around the atomics;
//   bwd_convert  dq = bf16(scale * dQ accumulator).
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdKeysPerWave = 32;
constexpr int kBwdBc = kBwdWaves * kBwdKeysPerWave;  // 128 keys per workgroup
constexpr int kBwdRowPad = 64;                       // dQ accumulator rows per head: multiple of this

// ---------------------------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic and LSE_i log2(e); zero the dQ accumulator row.  D/8 threads per row.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      const float* __restrict__ LSE, float* __restrict__ delta,
                                                      float* __restrict__ lse2, float* __restrict__ dqacc, int N,
                                                      int Npad, int64_t rows) {
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
      const int64_t prow = (row / N) * Npad + row % N;  // rows of a head are padded to Npad
      float4* z = (float4*)(dqacc + prow * D + part * 8);
      z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, TPR);
  if (row < rows && part == 0) {
    delta[row] = sum;
    if (lse2 != nullptr) lse2[row] = LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_convert_kernel(const float* __restrict__ acc, __bf16* __restrict__ dq,
                                                          float scale, int N, int Npad, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 8-element chunk of dq
  if (i >= n8) return;
  constexpr int CPR = D / 8;  // chunks per row
  const int64_t row = i / CPR;
  const int64_t prow = (row / N) * Npad + row % N;
  const float* a = acc + prow * D + (i % CPR) * 8;
  const float4 x = ((const float4*)a)[0];
  const float4 y = ((const float4*)a)[1];
  const bf16x4 lo = pack4(x.x * scale, x.y * scale, x.z * scale, x.w * scale);
  const bf16x4 hi = pack4(y.x * scale, y.y * scale, y.z * scale, y.w * scale);
  ((bf16x8*)dq)[i] = cat(lo, hi);
}

// ---------------------------------------------------------------------------------------------
// Query rows per tile of the main kernel: 32 at d=128 (keeps a wave's live state in its registers),
// 64 at d=64.  The dQ accumulator rows are padded to a multiple of 64, which covers both.
template <int D>
constexpr int bwd_rows_per_tile() { return D == 128 ? 32 : 64; }

// Byte offset of (key row, query col) in the dS^T tile [128 keys][BR queries] (bf16).  BR = 64:
// 128-byte rows with the tile swizzle.  BR = 32: 64-byte rows, four to a 256-byte bank range, so a
// transposing read (4 consecutive rows) is conflict-free as is; the 8-byte chunk index is XORed with
// row / 4 so that the per-key writes of 32 consecutive keys land on distinct banks.
template <int BR>
__device__ __forceinline__ uint32_t dst_off(int row, int col) {
  if constexpr (BR == 64) {
    return tile_off<64>(row, col);
  } else {
    return (uint32_t)(row * (BR * 2) + (((col >> 2) ^ ((row >> 2) & 7)) << 3) + ((col & 3) << 1));
  }
}

template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                          const float* __restrict__ LSE2,
                                                          const float* __restrict__ DELTA, float* __restrict__ dQacc,
                                                          __bf16* __restrict__ dK, __bf16* __restrict__ dV, int H,
                                                          int N, int Npad, float scale, float c_log2,
                                                          const int32_t* __restrict__ seqlens, int nkb, int BH) {
  constexpr int BR = bwd_rows_per_tile<D>();  // query rows per tile
  constexpr int QS = BR / 32;                 // 32-row halves of a tile
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int QTILE = BR * D * 2;           // bytes of a Q or dO tile
  constexpr int LOADS = BR * CH / 256;        // 16-byte loads per thread per tile and tensor
  constexpr int DS = D / 16;                  // k-steps over d
  constexpr int DT = D / 32;                  // 32-wide d tiles
  constexpr int STAGE = 2 * QTILE + 2 * 64 * 4;  // Q | dO | LSE log2 e (64 floats) | D (64 floats)
  constexpr int DST = kBwdBc * BR * 2;           // dS^T [128 keys][BR q] bf16
  constexpr int VALU_A = 16 * QS * 5;            // P and dS: 16 QS elements x (fma, exp, sub, mul, cvt)
  static_assert(QS * DT == kBwdWaves, "one 32x32 dQ tile per wave");
  // Separate, statically referenced LDS arrays (see the forward kernel): a direct load into one
  // stage is then never taken to alias the reads of another.
  __shared__ __attribute__((aligned(1024))) char st0_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char ds0_raw[DST];
  __shared__ __attribute__((aligned(1024))) char ds1_raw[DST];
  __shared__ __attribute__((aligned(1024))) char ds2_raw[DST];
  __shared__ __attribute__((aligned(1024))) char kst_raw[kBwdBc * D * 2];  // K of the block, [128][D]
  FA_LDS char* st0 = (FA_LDS char*)st0_raw;
  FA_LDS char* st1 = (FA_LDS char*)st1_raw;
  FA_LDS char* st2 = (FA_LDS char*)st2_raw;
  FA_LDS char* ds0 = (FA_LDS char*)ds0_raw;
  FA_LDS char* ds1 = (FA_LDS char*)ds1_raw;
  FA_LDS char* ds2 = (FA_LDS char*)ds2_raw;
  FA_LDS char* kst = (FA_LDS char*)kst_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;

  // ---- work item: (key block, batch*head); key block 0 has the most query tiles under the causal
  // mask, so ascending rank is heaviest first.  All key blocks of a head go to one XCD when B*H is
  // a multiple of 8 (its Q, dO and dQ accumulator rows then stay in that XCD's L2).
  const int wid = blockIdx.x;
  int kblock, bh;
  if ((BH & 7) == 0) {
    const int hpx = BH >> 3;
    const int j = wid >> 3;
    kblock = j / hpx;
    bh = (wid & 7) + 8 * (j - kblock * hpx);
  } else {
    kblock = wid / BH;
    bh = wid - kblock * BH;
  }
  const int b = bh / H;
  const int64_t row0 = (int64_t)bh * N;
  const __bf16* Qh = Q + row0 * D;
  const __bf16* Kh = K + row0 * D;
  const __bf16* Vh = V + row0 * D;
  const __bf16* dOh = dO + row0 * D;
  const float* LSEh = LSE2 + row0;
  const float* DELh = DELTA + row0;
  float* dQh = dQacc + (int64_t)bh * Npad * D;

  const int L = PADDED ? clamp_len(seqlens, b, N) : N;
  const int k0 = kblock * kBwdBc;
  const int kw = k0 + wave * kBwdKeysPerWave;
  const int my_key = kw + l32;

  f32x16 dvt[DT], dkt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dvt[dt] = zero16();
    dkt[dt] = zero16();
  }

  if (k0 < L) {
    // ---- stationary operands: K and V rows of this wave's keys (B operands of S and dP)
    bf16x8 kb[DS], vb[DS];
    {
      const int key = min(my_key, N - 1);  // keys past N are masked
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        kb[ds] = *(const bf16x8*)(Kh + (int64_t)key * D + 16 * ds + 8 * half);
        vb[ds] = *(const bf16x8*)(Vh + (int64_t)key * D + 16 * ds + 8 * half);
      }
    }
    // ---- K of the 128 keys staged in LDS: B operand of dQ = dS K, read transposed per k-step
    for (int p = threadIdx.x; p < kBwdBc * CH; p += 256) {
      const int r = p / CH, c = p % CH;
      const int key = min(k0 + r, N - 1);
      *(FA_LDS u32x4*)(kst + tile_off<D>(r, 8 * c)) = *(const u32x4*)(Kh + (int64_t)key * D + 8 * c);
    }
    // this wave's 32x32 dQ tile: queries 32 qsw + 0..31 of the tile, d = 32 dtq + 0..31
    const int qsw = wave / DT, dtq = wave % DT;
    const int dcol = 32 * dtq + 16 * (g16 & 1) + 4 * (j16 & 3);
    const int trow = 4 * (g16 >> 1) + (j16 >> 2);
    // per-lane LDS bases of the transposing reads of the dQ product (see the dQ phase)
    const uint32_t kb0 = tile_off<D>(trow, dcol), kb8 = tile_off<D>(trow + 8, dcol);
    uint32_t dsb[2][2];
#pragma unroll
    for (int par = 0; par < 2; ++par)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        dsb[par][hh] = dst_off<BR>(trow + 16 * par + 8 * hh, 32 * qsw + 16 * (g16 & 1) + 4 * (j16 & 3));

    const int nqt = (N + BR - 1) / BR;
    const int it0 = CAUSAL ? (k0 / BR) : 0;
    const int count = nqt - it0;  // query tiles this key block visits (>= 1)

    auto load_tile = [&](int u, FA_LDS char* dst) {
      const int qbase = (it0 + u) * BR;
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int slot = (n * kBwdWaves + wave) * 64;
        const int p = slot + lane;
        const int r = p / CH;
        const int c = (p % CH) ^ swz<D>(r);
        const int q = min(qbase + r, N - 1);
        gload_lds16(Qh + (int64_t)q * D + 8 * c, dst + slot * 16);
        gload_lds16(dOh + (int64_t)q * D + 8 * c, dst + QTILE + slot * 16);
      }
      if (wave < 2) {  // 64 rows of LSE log2 e / D; rows past the tile are clamped and unused
        const int q = min(qbase + lane, N - 1);
        gload_lds4(wave == 0 ? (const void*)(LSEh + q) : (const void*)(DELh + q), dst + 2 * QTILE + wave * 256);
      }
    };

    f32x16 s[QS], dp[QS];  // S and dP of the current tile: lane = key my_key, rows = queries
    // S = Q K^T and dP = dO V^T for the tile in st (A operands read row-major from LDS)
    auto scores = [&](const FA_LDS char* st) {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        s[qs] = zero16();
        dp[qs] = zero16();
      }
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          const uint32_t off = tile_off<D>(32 * qs + l32, 16 * ds + 8 * half);
          const bf16x8 qa = lds_read_b128(st, off);
          const bf16x8 da = lds_read_b128(st + QTILE, off);
          s[qs] = mfma32x32x16(qa, kb[ds], s[qs]);
          dp[qs] = mfma32x32x16(da, vb[ds], dp[qs]);
        }
      pipe_schedule<DS, 2 * QS, 2 * QS, 0, 2, 1>();  // fragment reads two k-steps ahead of their MFMAs
    };

    bf16x8 pb[2 * QS], db[2 * QS];  // P and dS packed (B operands of dV^T and dK^T), k = queries
    f32x16 accq = zero16();          // dQ tile of the previous query tile, added one iteration later

    // dQ(tile v) += accq: float atomics into the row-padded accumulator (unscaled).  Lane holds
    // d = 32 dtq + l32 and queries 8 g + 4 half + e of the wave's 32-row half; one base per g keeps
    // every offset an instruction immediate.
    auto add_dq = [&](int v) {
      float* base = dQh + (int64_t)((it0 + v) * BR + 32 * qsw + 4 * half) * D + 32 * dtq + l32;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int e = 0; e < 4; ++e) unsafeAtomicAdd(base + (8 * gq + e) * D, accq[4 * gq + e]);
    };

    // One tile: tile u in cur (Q, dO, LSE log2 e, D); st_next holds tile u+1; tile u+2 is loaded
    // into st_load.  dsw receives dS^T(u); dsr holds dS^T(u-1).
    auto step = [&](int u, const FA_LDS char* cur, const FA_LDS char* st_next, FA_LDS char* st_load,
                    FA_LDS char* dsw, const FA_LDS char* dsr) {
      wait_vmem();  // tile u+1 landed; the atomics issued one iteration ago have completed
      __syncthreads();
      if (u + 2 < count) load_tile(u + 2, st_load);
      if (u >= 2) add_dq(u - 2);  // issued now so that they too have a full iteration to complete
      const int qi0 = (it0 + u) * BR;
      const bool has = u < count;

      // ---- hidden pairs (causal diagonal, key padding, ragged tail): scores to -inf, scaled domain
      float cf = c_log2;
      if (has && ((kw + kBwdKeysPerWave > L) || (qi0 + BR > N) || (CAUSAL && kw + kBwdKeysPerWave - 1 > qi0))) {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int query = qi0 + 32 * qs + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool vis = (my_key < L) & (query < N) & (!CAUSAL | (my_key <= query));
            s[qs][r] = vis ? s[qs][r] * c_log2 : -INFINITY;
          }
        cf = 1.f;
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- A: dQ(u-1) on the matrix cores || P(u), dS(u) on the VALU
      const FA_LDS float* lse_t = (const FA_LDS float*)(cur + 2 * QTILE);
      const FA_LDS float* del_t = lse_t + 64;
#pragma unroll
      for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int qloc = 32 * qs + 8 * gq + 4 * half;
          const f32x4 lse4 = *(const FA_LDS f32x4*)(lse_t + qloc);
          const f32x4 del4 = *(const FA_LDS f32x4*)(del_t + qloc);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * gq + e;
            const float p = fast_exp2(fmaf(s[qs][r], cf, -lse4[e]));
            s[qs][r] = p;
            dp[qs][r] = p * (dp[qs][r] - del4[e]);
          }
        }
#pragma unroll
      for (int ks = 0; ks < 2 * QS; ++ks) {
        pb[ks] = pack8(s[ks >> 1], 8 * (ks & 1));
        db[ks] = pack8(dp[ks >> 1], 8 * (ks & 1));
      }
      accq = zero16();
#pragma unroll
      for (int ks = 0; ks < kBwdBc / 16; ++ks) {
        // dS^T rows trow + 16 ks and trow + 16 ks + 8 (per-lane bases for the parity of ks and the
        // +8: the swizzles repeat every 32 rows of dS^T and 16 rows of K)
        const uint32_t srow = dsb[ks & 1][0] + (ks >> 1) * 32 * BR * 2;
        const uint32_t srow8 = dsb[ks & 1][1] + (ks >> 1) * 32 * BR * 2;
        const bf16x8 sa = cat(lds_read_tr(dsr, srow), lds_read_tr(dsr, srow8));
        const bf16x8 kq = cat(lds_read_tr(kst, kb0 + ks * 16 * D * 2), lds_read_tr(kst, kb8 + ks * 16 * D * 2));
        accq = mfma32x32x16(sa, kq, accq);
      }
      pipe_schedule<kBwdBc / 16, 4, 1, VALU_A / (kBwdBc / 16), 2, 0>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2 * QS; ++ks) asm volatile("" : "+v"(pb[ks]), "+v"(db[ks]));

      // dS^T(u) -> LDS [key][q] (bf16): db[ks] holds queries 16 ks + 4 half + 0..3 and 16 ks + 8 + 4 half + 0..3
#pragma unroll
      for (int ks = 0; ks < 2 * QS; ++ks) {
        const int qloc = 16 * ks + 4 * half;
        *(FA_LDS bf16x4*)(dsw + dst_off<BR>(32 * wave + l32, qloc)) = __builtin_shufflevector(db[ks], db[ks], 0, 1, 2, 3);
        *(FA_LDS bf16x4*)(dsw + dst_off<BR>(32 * wave + l32, qloc + 8)) = __builtin_shufflevector(db[ks], db[ks], 4, 5, 6, 7);
      }
      if (!has) return;

      // ---- B: dV^T += dO^T P ; dK^T += Q^T dS  (A operands through the transposing read)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t tb0 = tile_off<D>(trow, 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3));
        const uint32_t tb8 = tile_off<D>(trow + 8, 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3));
#pragma unroll
        for (int ks = 0; ks < 2 * QS; ++ks) {
          const bf16x8 da = cat(lds_read_tr(cur + QTILE, tb0 + ks * 16 * D * 2), lds_read_tr(cur + QTILE, tb8 + ks * 16 * D * 2));
          const bf16x8 qa = cat(lds_read_tr(cur, tb0 + ks * 16 * D * 2), lds_read_tr(cur, tb8 + ks * 16 * D * 2));
          dvt[dt] = mfma32x32x16(da, pb[ks], dvt[dt]);
          dkt[dt] = mfma32x32x16(qa, db[ks], dkt[dt]);
        }
      }
      pipe_schedule<2 * QS * DT, 4, 2, 0, 2, 2>();
      __builtin_amdgcn_sched_barrier(0);

      // ---- C: S(u+1), dP(u+1)
      if (u + 1 < count) scores(st_next);
    };

    load_tile(0, st0);
    if (count > 1) load_tile(1, st1);
    wait_vmem();
    __syncthreads();
    scores(st0);
    for (int u = 0; u <= count; u += 3) {
      step(u, st0, st1, st2, ds0, ds2);
      if (u + 1 <= count) step(u + 1, st1, st2, st0, ds1, ds0);
      if (u + 2 <= count) step(u + 2, st2, st0, st1, ds2, ds1);
    }
    add_dq(count - 1);  // dQ of the last tile, computed in the drain iteration
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
hipError_t launch_main(const Problem& p, const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                       const float* delta, float* dqacc, void* dk, void* dv) {
  const int nkb = (p.N + kBwdBc - 1) / kBwdBc;
  const int BH = p.B * p.H;
  const int Npad = bwd_rows_padded(p.N);
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, PADDED>), dim3((unsigned)(nkb * BH)), dim3(256), 0, p.stream,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, lse2, delta, dqacc,
                     (__bf16*)dk, (__bf16*)dv, p.H, p.N, Npad, p.scale, p.scale * kLog2e, p.seqlens, nkb, BH);
  return hipGetLastError();
}

template <int D, typename T>
hipError_t launch_pre(const Problem& p, const void* o, const void* dO, const float* lse, float* delta, float* lse2,
                      float* dqacc) {
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  constexpr int rows_per_block = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D, T>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(256), 0, p.stream, (const T*)o, (const T*)dO, lse, delta, lse2, dqacc, p.N,
                     bwd_rows_padded(p.N), rows);
  return hipGetLastError();
}

}  // namespace

int bwd_rows_padded(int N) { return (N + kBwdRowPad - 1) / kBwdRowPad * kBwdRowPad; }
int64_t bwd_bf16_grid(int B, int H, int N) { return (int64_t)((N + kBwdBc - 1) / kBwdBc) * B * H; }

hipError_t launch_bwd_prepare(const Problem& p, bool bf16, const void* o, const void* dO, const float* lse,
                              void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, bf16);
  float* delta = (float*)((char*)workspace + ws.delta_off);
  if (bf16) {
    float* lse2 = (float*)((char*)workspace + ws.lse2_off);
    float* dqacc = (float*)((char*)workspace + ws.dqacc_off);
    return p.d == 64 ? launch_pre<64, __bf16>(p, o, dO, lse, delta, lse2, dqacc)
                     : launch_pre<128, __bf16>(p, o, dO, lse, delta, lse2, dqacc);
  }
  return p.d == 64 ? launch_pre<64, float>(p, o, dO, lse, delta, nullptr, nullptr)
                   : launch_pre<128, float>(p, o, dO, lse, delta, nullptr, nullptr);
}

hipError_t launch_bwd_main_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                                void* dk, void* dv, void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, true);
  const float* delta = (const float*)((char*)workspace + ws.delta_off);
  const float* lse2 = (const float*)((char*)workspace + ws.lse2_off);
  float* dqacc = (float*)((char*)workspace + ws.dqacc_off);
  const bool pad = p.seqlens != nullptr;
  if (p.d == 64) {
    if (p.causal)
      return pad ? launch_main<64, true, true>(p, q, k, v, dO, lse2, delta, dqacc, dk, dv)
                 : launch_main<64, true, false>(p, q, k, v, dO, lse2, delta, dqacc, dk, dv);
    return pad ? launch_main<64, false, true>(p, q, k, v, dO, lse2, delta, dqacc, dk, dv)
               : launch_main<64, false, false>(p, q, k, v, dO, lse2, delta, dqacc, dk, dv);
  }
  if (p.causal)
    return pad ? launch_main<128, true, true>(p, q, k, v, dO, lse2, delta, dqacc, dk, dv)
               : launch_main<128, true, false>(p, q, k, v, dO, lse2, delta, dqacc, dk, dv);
  return pad ? launch_main<128, false, true>(p, q, k, v, dO, lse2, delta, dqacc, dk, dv)
             : launch_main<128, false, false>(p, q, k, v, dO, lse2, delta, dqacc, dk, dv);
}

hipError_t launch_bwd_finish_bf16(const Problem& p, void* dq, void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, true);
  const float* dqacc = (const float*)((char*)workspace + ws.dqacc_off);
  const int64_t n8 = (int64_t)p.B * p.H * p.N * p.d / 8;
  const int Npad = bwd_rows_padded(p.N);
  if (p.d == 64)
    hipLaunchKernelGGL((bwd_convert_kernel<64>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, p.stream, dqacc,
                       (__bf16*)dq, p.scale, p.N, Npad, n8);
  else
    hipLaunchKernelGGL((bwd_convert_kernel<128>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, p.stream, dqacc,
                       (__bf16*)dq, p.scale, p.N, Npad, n8);
  return hipGetLastError();
}

}  // namespace fa
