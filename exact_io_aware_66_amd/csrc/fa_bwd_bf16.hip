// Backward of exact attention: the row statistics and dK, dV; bf16 inputs, fp32 accumulation, on
// gfx950 matrix cores.
//
// The backward never reads a stored N x N matrix: it recomputes each block of probabilities from
// Q, K and the per-row log-sum-exp the forward kept (NOTE-005: FlashAttention, "Method" and "Key
// components"; aicassindra FlashAttention architecture page, "The architecture: every piece
// explained").  The gradient formulas are the chain rule through softmax for the loss sum(dO*O):
//   P = exp(S - LSE),  dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//   dS = P * (dP - D),  dK = scale dS^T Q,  dQ = scale dS K.
//
// Kernels here:
//   bwd_pre   -D_i and LSE_i log2(e) (fp32) into the workspace;
//   bwd_dkdv  one workgroup per 128 keys of a (batch, head): 4 waves x 32 keys, one per SIMD (d = 128:
//             one workgroup per compute unit; d = 64: two, so two waves per SIMD).
//             K and V of the wave stay in registers (B operands of S = Q K^T and dP = dO V^T), and
//             dK^T, dV^T accumulate in registers over the whole walk of query tiles of 32 rows.
//             The query tiles (Q, dO, LSE log2 e, -D) stream through a
//             four-stage LDS ring filled by direct global->LDS loads three tiles ahead.  Per tile u,
//             one barrier, then
//               C: S(u+1) = Q K^T and dP(u+1) - D = dO V^T - D on the matrix cores (into the
//                  other of two register sets; the dP accumulators start from -D), interleaved with
//                  P(u) = exp2(S scale log2 e - LSE log2 e), dS(u) = P (dP - D) and their packing
//                  to bf16 for the first half of the queries;
//               B: dV^T += dO^T P(u), dK^T += Q^T dS(u) (dO^T, Q^T through transposing LDS reads),
//                  first-half queries first, interleaved with P and dS of the second half.
//             Tiles with hidden pairs (causal diagonal, key padding, ragged tail) set the hidden
//             scores to -inf first (so P = 0 and dS = 0 there).
// At d = 128 without a block mask (dense, or with dropout) the dK/dV pass runs bwd_dkdv_kl_kernel
// (fa_bwd_dkdv_kl.hip) instead: the same arithmetic in the same order with K in LDS, so that two
// waves share each SIMD; bwd_dkdv_kernel serves d = 64 and the block-sparse masks.
// dQ comes from a query-block-outer kernel of its own (fa_bwd_dq.hip), so that every output row has
// exactly one writer and no atomic additions are needed anywhere in the backward.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdKeysPerWave = 32;
constexpr int kBwdBc = kBwdWaves * kBwdKeysPerWave;  // 128 keys per workgroup
#ifndef FA_BWD_READ_AHEAD
#define FA_BWD_READ_AHEAD 0
#endif
#ifndef FA_BWD_READ_AHEAD_B
#define FA_BWD_READ_AHEAD_B 0
#endif
// LDS operand fragments are read this many MFMA steps ahead: row reads (score phase) and
// transposing reads (dV/dK phase); 0 selects the measured choice per head size (d = 64: one and
// three, -0.5 to -1.4 % dK/dV time against two and two; d = 128: two and two)
template <int D>
constexpr int bwd_ra() { return FA_BWD_READ_AHEAD > 0 ? FA_BWD_READ_AHEAD : D == 64 ? 1 : 2; }
template <int D>
constexpr int bwd_rb() { return FA_BWD_READ_AHEAD_B > 0 ? FA_BWD_READ_AHEAD_B : D == 64 ? 3 : 2; }

// ---------------------------------------------------------------------------------------------
// -D_i = -sum_c dO_ic O_ic and (bf16 path) LSE_i log2(e).  D/8 threads per row.  The workspace keeps
// the negated statistic: the dK/dV pass starts its dP accumulation from it, so the products come
// out as dP - D directly.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      const float* __restrict__ LSE, float* __restrict__ delta,
                                                      float* __restrict__ lse2, int64_t rows) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float sum = 0.f;
  if (row < rows) {
    const T* o = O + row * D + part * 8;
    const T* g = dO + row * D + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) sum = fmaf((float)o[e], (float)g[e], sum);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, TPR);
  if (row < rows && part == 0) {
    delta[row] = -sum;
    if (lse2 != nullptr) lse2[row] = LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------------------------
// Query rows per tile of the dK/dV kernel: 32.  At d = 64 that keeps a wave within 256 registers
// (no accumulator registers needed), so two workgroups share a compute unit and each SIMD runs two
// waves that cover each other's stalls: measured 17-24 % faster than 64-row tiles with one
// workgroup per compute unit, bitwise the same results.  At d = 128 a wave needs about 400 registers
// (dK^T and dV^T accumulators, K and V, two sets of S and dP), one workgroup per compute unit.
template <int D>
constexpr int bwd_rows_per_tile() { return 32; }
template <int D>
constexpr int bwd_wg_per_cu() { return D == 64 ? 2 : 1; }

template <int D, bool CAUSAL, bool PADDED, bool SPARSE, bool DROP>
__global__ __launch_bounds__(256, bwd_wg_per_cu<D>()) void bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                          const float* __restrict__ LSE2,
                                                          const float* __restrict__ DELTA, __bf16* __restrict__ dK,
                                                          __bf16* __restrict__ dV, int H, int N, float scale,
                                                          float c_log2, const int32_t* __restrict__ seqlens,
                                                          const uint8_t* __restrict__ bmask, Dropout dr, int BH) {
  constexpr int kRA = bwd_ra<D>();
  constexpr int kRB = bwd_rb<D>();
  constexpr int BR = bwd_rows_per_tile<D>();  // query rows per tile
  constexpr int QS = BR / 32;                 // 32-row halves of a tile
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int QTILE = BR * D * 2;           // bytes of a Q or dO tile
  constexpr int LOADS = BR * CH / 256;        // 16-byte loads per thread per tile and tensor
  constexpr int DS = D / 16;                  // k-steps over d
  constexpr int DT = D / 32;                  // 32-wide d tiles
  constexpr int STAGE = 2 * QTILE + 4 * 256;  // Q | dO | per-wave row statistics: LSE log2 e, D, LSE, D
  constexpr int VMEM_PER_TILE = 2 * LOADS + 1;  // vector-memory instructions per wave per tile
  // Leading query tiles that cross the causal diagonal of the block's 128 keys; every later tile is
  // fully visible to every key of the block.
  constexpr int HEAD = CAUSAL ? kBwdBc / BR : 0;
  // Four separate, statically referenced LDS stages (as in the forward kernel, a direct load into one
  // stage is then never taken to alias the reads of another): tile u lives in stage u % 4.
  __shared__ __attribute__((aligned(1024))) char st0_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char st3_raw[STAGE];
  // block-sparse: the visible query tiles of this key block, in order (kBwdBc / BR per mask block)
  __shared__ uint16_t tlist_raw[SPARSE ? (kBwdBc / BR) * kMaxMaskBlocks : 1];
  __shared__ int tcount_raw;
  // dropout: per wave, the keep bytes of each 32 x 32 (query, key) block of a tile, key-major
  __shared__ __attribute__((aligned(16))) uint8_t drop_raw[DROP ? kBwdWaves * QS * 1024 : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;

  // ---- work item: (key block, batch*head); key block 0 has the most query tiles under the causal
  // mask, so ascending rank is heaviest first.  All key blocks of a head go to one XCD when B*H is
  // a multiple of 8 (its Q and dO rows then stay in that XCD's L2).
  const int wid = work_item();
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
      const int key = min(my_key, N - 1);  // keys past N are never written back
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        kb[ds] = *(const bf16x8*)(Kh + (int64_t)key * D + 16 * ds + 8 * half);
        vb[ds] = *(const bf16x8*)(Vh + (int64_t)key * D + 16 * ds + 8 * half);
      }
    }
    const int trow = 4 * (g16 >> 1) + (j16 >> 2);

    const int nqt = (N + BR - 1) / BR;
    const int it0 = CAUSAL ? (k0 / BR) : 0;
    int count = nqt - it0;  // query tiles this key block visits (>= 1)
    // Block-sparse: the steps walk the list of visible query tiles (in tile order); the masked head
    // (the causal diagonal block) is present only when that block is visible, and then it is the
    // list's head, tiles it0 .. it0+HEAD-1 as in the dense walk.
    const FA_LDS uint16_t* const tlist = (const FA_LDS uint16_t*)tlist_raw;
    bool head_visible = true;
    if constexpr (SPARSE) {
      const int nb = (N + kMaskBlock - 1) / kMaskBlock;
      const uint8_t* bcol = bmask + (int64_t)bh * nb * nb + kblock;
      if (wave == 0)
        compact_tiles<kBwdBc / BR>((FA_LDS uint16_t*)tlist_raw, (FA_LDS int*)&tcount_raw, it0 * BR / kMaskBlock, nb,
                                   nqt, [&](int qb) { return bcol[(int64_t)qb * nb] != 0 ? 1 : 0; });
      __syncthreads();
      count = *(volatile FA_LDS int*)&tcount_raw;
      head_visible = CAUSAL && count > 0 && list_tile(tlist[0]) == it0;
    }

    // Tile loads: buffer loads straight into LDS.  Rows past N read as zeros (the buffer ends at the
    // head's last row), and a zero Q and dO row adds exactly nothing to dK and dV, so the ragged last
    // tile needs no mask.  Per-lane byte offsets inside a tile are loop-invariant.
    uint32_t voff[LOADS];
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int p = (n * kBwdWaves + wave) * 64 + lane;
      const int r = p / CH;
      const int c = (p % CH) ^ swz<D>(r);
      voff[n] = (uint32_t)(r * D + 8 * c) * 2;
    }
    // Wave w fetches 64 rows of statistic w & 1 (0: LSE log2 e, 1: D) into its own 256-byte slot.
    const float* stat = (wave & 1) ? DELTA + row0 : LSE2 + row0;
    // One buffer resource per tensor over the whole head (built once): a tile's byte offset goes into
    // the per-lane offset, which the range check covers, so rows past N still read as zeros.
    const u32x4 rq = make_rsrc(Qh, N * D * 2);
    const u32x4 rg = make_rsrc(dOh, N * D * 2);
    const u32x4 rs = make_rsrc(stat, N * 4);
    auto load_tile = [&](int u, FA_LDS char* dst) {
      const int qbase = (SPARSE ? list_tile(tlist[u]) : it0 + u) * BR;
      const uint32_t tb = (uint32_t)qbase * D * 2;
#pragma unroll
      for (int n = 0; n < LOADS; ++n) {
        const int slot = (n * kBwdWaves + wave) * 64;
        const uint32_t off = voff[n] + tb;
        bload_lds16(rq, off, dst + slot * 16);
        bload_lds16(rg, off, dst + QTILE + slot * 16);
      }
      bload_lds4(rs, (uint32_t)(qbase + lane) * 4, dst + 2 * QTILE + wave * 256);
    };

    // S and dP of two consecutive tiles (set u % 2 holds tile u): lane = key my_key, rows = queries
    f32x16 s[2][QS], dp[2][QS];

    // S = Q K^T and dP = dO V^T for the tile in st into set P, DS k-steps of 2 QS MFMAs.  The A
    // operands are read row-major from LDS two k-steps ahead (a ring of three fragment sets);
    // `between(ds)` places other work after the MFMAs of k-step ds.
    auto scores = [&](auto par, const FA_LDS char* st, auto&& between) __attribute__((always_inline)) {
      constexpr int P = decltype(par)::value;
      bf16x8 fq[kRA + 1][QS], fd[kRA + 1][QS];
      auto rd = [&](int ds, bf16x8 (&q)[QS], bf16x8 (&d)[QS]) {
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          const uint32_t off = tile_off<D>(32 * qs + l32, 16 * ds + 8 * half);
          q[qs] = lds_read_b128(st, off);
          d[qs] = lds_read_b128(st + QTILE, off);
        }
      };
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        s[P][qs] = zero16();
        // dP starts from -D of the tile's rows (the workspace's statistic, in the accumulator layout:
        // element 4 gq + e is query 32 qs + 8 gq + 4 half + e), so it accumulates dP - D.  With
        // dropout it starts from -D t / 256 instead: a kept element's dP is scaled by 256 / t, which
        // gives (256 / t) dP - D (and with t = 256 exactly the dense values).
        const FA_LDS float* nd = (const FA_LDS float*)(st + 2 * QTILE) + 64 + 32 * qs + 4 * half;
        const f32x4 a = *(const FA_LDS f32x4*)(nd), b = *(const FA_LDS f32x4*)(nd + 8);
        const f32x4 c = *(const FA_LDS f32x4*)(nd + 16), d = *(const FA_LDS f32x4*)(nd + 24);
        dp[P][qs] = __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7),
                                            __builtin_shufflevector(c, d, 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2, 3, 4, 5,
                                            6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        if constexpr (DROP) dp[P][qs] *= (float)dr.t * (1.f / 256.f);
      }
#pragma unroll
      for (int ds = 0; ds < kRA && ds < DS; ++ds) rd(ds, fq[ds], fd[ds]);
      // At d = 64 (two workgroups per compute unit, whose waves drift apart) the wave that feeds its
      // score products to the matrix cores goes first: -3 to -5 % dK/dV time (measured)
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        __builtin_amdgcn_sched_barrier(0);
        if (ds + kRA < DS) rd(ds + kRA, fq[(ds + kRA) % (kRA + 1)], fd[(ds + kRA) % (kRA + 1)]);
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          s[P][qs] = mfma32x32x16(fq[ds % (kRA + 1)][qs], kb[ds], s[P][qs]);
          dp[P][qs] = mfma32x32x16(fd[ds % (kRA + 1)][qs], vb[ds], dp[P][qs]);
        }
        between(ds);
      }
      if constexpr (D == 64) __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    };

    bf16x8 pb[2 * QS], db[2 * QS];  // P and dS packed (B operands of dV^T and dK^T), k = queries

    // One tile u (set P = u % 2, in stage cur; tile u+1 in stage nxt; tile u+3 is loaded into
    // stage ldst).  MASK: tile u crosses the causal diagonal of this block.  Every instance is
    // straight-line code: which tiles take the masked form is decided outside the loop.
    auto step = [&](auto mask, auto par, int u, const FA_LDS char* cur, const FA_LDS char* nxt, FA_LDS char* ldst)
        __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask)::value;
      constexpr int P = decltype(par)::value;
      // tile u+1 must have landed; tile u+2 (issued one step ago) may still be in flight
      if (u + 2 < count) wait_vmem_n<VMEM_PER_TILE>();
      else wait_vmem();
      barrier();
      if (u + 3 < count) load_tile(u + 3, ldst);

      // Dropout keep words of tile u in this kernel's layout (lane = key, 16 queries per 32-row half):
      // each lane draws the words of one query (the layout the generator is defined in), writes the
      // bytes key-major into the wave's LDS block and reads back the 4 words of its own key.
      u32x4 kwt[QS];
      if constexpr (DROP) {
        const int qb0 = (SPARSE ? list_tile(tlist[u]) : it0 + u) * BR;
        FA_LDS uint8_t* mt = (FA_LDS uint8_t*)drop_raw + wave * QS * 1024;
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
          const u32x4 w = dropout_words(dr, (uint32_t)bh, qb0 + 32 * qs + l32, kw / 32, half);
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) mt[qs * 1024 + (8 * g + 4 * half + e) * 32 + l32] = (uint8_t)(w[g] >> (8 * e));
        }
#pragma unroll
        for (int qs = 0; qs < QS; ++qs)
#pragma unroll
          for (int g = 0; g < 4; ++g) kwt[qs][g] = *(const FA_LDS uint32_t*)(mt + qs * 1024 + l32 * 32 + 8 * g + 4 * half);
      }

      float cf = c_log2;
      if constexpr (MASK) {  // hidden pairs (key > query) to -inf, in the scaled domain
        const int qi0 = (it0 + u) * BR;
#pragma unroll
        for (int qs = 0; qs < QS; ++qs)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int query = qi0 + 32 * qs + 8 * (r >> 2) + 4 * half + (r & 3);
            s[P][qs][r] = (my_key <= query) ? s[P][qs][r] * c_log2 : -INFINITY;
          }
        cf = 1.f;
      }

      // ---- C: S(u+1), dP(u+1) on the matrix cores || P(u), dS(u) on the VALU, then packed
      const FA_LDS float* lse_t = (const FA_LDS float*)(cur + 2 * QTILE);
      const FA_LDS float* del_t = lse_t + 64;
      // LSE log2 e (and, with dropout, -D) of the lane's 4 queries in each 8-query group gq of each
      // 32-row half qs
      f32x4 lse4[QS][4], nd4[QS][DROP ? 4 : 1];
#pragma unroll
      for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          lse4[qs][gq] = *(const FA_LDS f32x4*)(lse_t + 32 * qs + 8 * gq + 4 * half);
          if constexpr (DROP) nd4[qs][gq] = *(const FA_LDS f32x4*)(del_t + 32 * qs + 8 * gq + 4 * half);
        }
      // work unit e of k-step ks (16 queries; e < 4: two elements of P and dS, e = 4: the packing)
      auto unit = [&](int ks, int e) {
        const int qs = ks >> 1;
        if (e < 4) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int r = 8 * (ks & 1) + 2 * e + h;
            const float p = fast_exp2(fmaf(s[P][qs][r], cf, -lse4[qs][r >> 2][r & 3]));
            float dpv = dp[P][qs][r];  // dP - D (dropout: dP - D t / 256)
            float pv = p;  // P for dV: the kept probabilities (their 256/t scale is applied to dV at the end)
            if constexpr (DROP) {
              const bool keep = ((kwt[qs][r >> 2] >> (8 * (r & 3))) & 0xFFu) < dr.t;
              dpv = keep ? dpv * dr.scale : nd4[qs][r >> 2][r & 3];  // (256 / t) dP - D, or 0 - D
              pv = keep ? p : 0.f;
            }
            s[P][qs][r] = pv;
            dp[P][qs][r] = p * dpv;
          }
        } else {
          pb[ks] = pack8(s[P][qs], 8 * (ks & 1));
          db[ks] = pack8(dp[P][qs], 8 * (ks & 1));
        }
      };
      // The VALU work in query order, 5 units per k-step: the first half of the queries beside the
      // score MFMAs of tile u+1, the second half beside the dV/dK MFMAs of the first half (which do
      // not need it), each spread evenly, so both matrix-core phases carry VALU work.
      constexpr int HALF = 5 * QS;  // units per half
      auto spread = [&](int base, int step, int steps) {  // the units of this step of a phase
#pragma unroll
        for (int x = 0; x < HALF; ++x)
          if (x * steps / HALF == step) unit(base + x / 5, x % 5);
      };
      // B-phase operands: dO^T and Q^T of tile u through the transposing read, kRB steps ahead in a
      // ring; the first kRB are read during the last two k-steps of the score products, so the
      // matrix cores do not wait for them at the phase change
      constexpr int BS = DT * 2 * QS;  // steps (ks, dt) of 2 MFMAs
      bf16x8 bd[kRB + 1], bq[kRB + 1];
      auto rdb = [&](int i, bf16x8& d, bf16x8& q) {
        const int ks = i / DT, dt = i % DT;
        const uint32_t tb0 = tile_off<D>(trow, 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3)) + ks * 16 * D * 2;
        const uint32_t tb8 = tile_off<D>(trow + 8, 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3)) + ks * 16 * D * 2;
        d = cat(lds_read_tr(cur + QTILE, tb0), lds_read_tr(cur + QTILE, tb8));
        q = cat(lds_read_tr(cur, tb0), lds_read_tr(cur, tb8));
      };
      auto valu_c = [&](int ds) {
        spread(0, ds, DS);
        if (ds == DS - 2) {
#pragma unroll
          for (int i = 0; i < kRB && i < BS; ++i) rdb(i, bd[i], bq[i]);
        }
      };
      // (after the last tile the product reads a stale or unwritten stage; its result is unused)
      scores(std::integral_constant<int, 1 - P>{}, nxt, valu_c);

      // ---- B: dV^T += dO^T P ; dK^T += Q^T dS  (A operands through the transposing read), k-steps
      // of queries outermost
#pragma unroll
      for (int i = 0; i < BS; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + kRB < BS) rdb(i + kRB, bd[(i + kRB) % (kRB + 1)], bq[(i + kRB) % (kRB + 1)]);
        const int ks = i / DT, dt = i % DT;
        dvt[dt] = mfma32x32x16(bd[i % (kRB + 1)], pb[ks], dvt[dt]);
        dkt[dt] = mfma32x32x16(bq[i % (kRB + 1)], db[ks], dkt[dt]);
        if (i < DT * QS) spread(QS, i, DT * QS);
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    FA_LDS char* const st[4] = {(FA_LDS char*)st0_raw, (FA_LDS char*)st1_raw, (FA_LDS char*)st2_raw,
                                (FA_LDS char*)st3_raw};
    // step u with the stage ring and the score set of phase PH = u % 4 (all compile-time)
    auto at = [&](auto mask, auto ph, int u) __attribute__((always_inline)) {
      constexpr int PH = decltype(ph)::value;
      step(mask, std::integral_constant<int, PH % 2>{}, u, st[PH], st[(PH + 1) % 4], st[(PH + 3) % 4]);
    };
    using M = std::true_type;
    using C = std::false_type;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    // fully visible tiles from u on, four per iteration so that stages and score sets stay
    // compile-time (the walk starts in phase PH0 = u % 4)
    auto visible_tiles = [&](auto ph0, int u) __attribute__((always_inline)) {
      constexpr int PH0 = decltype(ph0)::value;
      for (; u + 3 < count; u += 4) {
        at(C{}, std::integral_constant<int, PH0>{}, u);
        at(C{}, std::integral_constant<int, (PH0 + 1) % 4>{}, u + 1);
        at(C{}, std::integral_constant<int, (PH0 + 2) % 4>{}, u + 2);
        at(C{}, std::integral_constant<int, (PH0 + 3) % 4>{}, u + 3);
      }
      if (u < count) at(C{}, std::integral_constant<int, PH0>{}, u);
      if (u + 1 < count) at(C{}, std::integral_constant<int, (PH0 + 1) % 4>{}, u + 1);
      if (u + 2 < count) at(C{}, std::integral_constant<int, (PH0 + 2) % 4>{}, u + 2);
    };

    if (!SPARSE || count > 0) {
      load_tile(0, st[0]);
      if (count > 1) load_tile(1, st[1]);
      if (count > 2) load_tile(2, st[2]);
      wait_vmem();
      barrier();
      scores(I0{}, st[0], [](int) {});

      if (!SPARSE || head_visible || !CAUSAL) {
        // masked head (causal): tiles 0 .. HEAD-1
        if constexpr (HEAD >= 1) at(M{}, I0{}, 0);
        if constexpr (HEAD >= 2) { if (count > 1) at(M{}, I1{}, 1); }
        if constexpr (HEAD >= 3) { if (count > 2) at(M{}, I2{}, 2); }
        if constexpr (HEAD >= 4) { if (count > 3) at(M{}, I3{}, 3); }
        visible_tiles(std::integral_constant<int, HEAD % 4>{}, HEAD);
      } else {
        visible_tiles(I0{}, 0);  // (block-sparse, causal) the diagonal block is masked out: no head
      }
    }
  }

  // ---- dK = scale dS^T Q, dV: lane holds key my_key, d = 32 dt + 8 gq + 4 half + 0..3.  Keys at
  // or past the valid length are hidden from every query: their gradients are zero (selected, not
  // multiplied: their unmasked accumulators may hold any value).  A store of the accumulator layout
  // would write 8-byte pieces of 32 rows per instruction; instead each wave stages its 32 rows of dK
  // and dV in its own LDS stage (256-byte rows, the tile swizzle) and writes them back as whole
  // 16-byte chunks, 64 / CH full rows per instruction.
  static_assert(2 * kBwdKeysPerWave * D * 2 <= STAGE, "a wave's dK and dV rows fit in one LDS stage");
  barrier();  // every wave is done with the stages of the query tiles
  {
    FA_LDS char* const ep = wave == 0 ? (FA_LDS char*)st0_raw
                            : wave == 1 ? (FA_LDS char*)st1_raw
                            : wave == 2 ? (FA_LDS char*)st2_raw : (FA_LDS char*)st3_raw;
    constexpr int VB = kBwdKeysPerWave * D * 2;  // bytes of the wave's dK rows (dV rows follow)
    const bool live = (!PADDED || my_key < L) && my_key < N;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dt + 8 * gq + 4 * half;
        float kx[4], vx[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[e] = live ? dkt[dt][4 * gq + e] * scale : 0.f;
          vx[e] = live ? dvt[dt][4 * gq + e] * (DROP ? dr.scale : 1.f) : 0.f;
        }
        *(FA_LDS bf16x4*)(ep + tile_off<D>(l32, d0)) = pack4(kx[0], kx[1], kx[2], kx[3]);
        *(FA_LDS bf16x4*)(ep + VB + tile_off<D>(l32, d0)) = pack4(vx[0], vx[1], vx[2], vx[3]);
      }
    constexpr int CHUNKS = kBwdKeysPerWave * CH / 64;  // 16-byte chunks per lane and tensor
#pragma unroll
    for (int n = 0; n < CHUNKS; ++n) {
      const int pch = n * 64 + lane;
      const int r = pch / CH, c = pch % CH;
      const int key = kw + r;
      const bf16x8 kv = lds_read_b128(ep, tile_off<D>(r, 8 * c));
      const bf16x8 vv = lds_read_b128(ep + VB, tile_off<D>(r, 8 * c));
      if (key < N) {
        *(bf16x8*)(dK + (row0 + key) * D + 8 * c) = kv;
        *(bf16x8*)(dV + (row0 + key) * D + 8 * c) = vv;
      }
    }
  }
}

template <int D, bool CAUSAL, bool PADDED, bool SPARSE, bool DROP>
hipError_t launch_dkdv(const Problem& p, const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                       const float* delta, void* dk, void* dv) {
  const int nkb = (p.N + kBwdBc - 1) / kBwdBc;
  const int BH = p.B * p.H;
  const Dropout dr{p.drop_k0, p.drop_k1, p.drop_off2, p.drop_t, 256.f / (float)p.drop_t};
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, PADDED, SPARSE, DROP>), dim3((unsigned)(nkb * BH)), dim3(256), 0,
                     p.stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, lse2, delta,
                     (__bf16*)dk, (__bf16*)dv, p.H, p.N, p.scale, p.scale * kLog2e, p.seqlens, p.block_mask, dr, BH);
  return hipGetLastError();
}

template <int D, bool SPARSE, bool DROP>
hipError_t launch_dkdv_m(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                         const float* lse2, const float* delta, void* dk, void* dv) {
  const bool pad = p.seqlens != nullptr;
  if (p.causal)
    return pad ? launch_dkdv<D, true, true, SPARSE, DROP>(p, q, k, v, dO, lse2, delta, dk, dv)
               : launch_dkdv<D, true, false, SPARSE, DROP>(p, q, k, v, dO, lse2, delta, dk, dv);
  return pad ? launch_dkdv<D, false, true, SPARSE, DROP>(p, q, k, v, dO, lse2, delta, dk, dv)
             : launch_dkdv<D, false, false, SPARSE, DROP>(p, q, k, v, dO, lse2, delta, dk, dv);
}

template <int D>
hipError_t launch_dkdv_d(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                         const float* lse2, const float* delta, void* dk, void* dv) {
  if (p.dropout) return launch_dkdv_m<D, false, true>(p, q, k, v, dO, lse2, delta, dk, dv);
  return p.block_mask != nullptr ? launch_dkdv_m<D, true, false>(p, q, k, v, dO, lse2, delta, dk, dv)
                                 : launch_dkdv_m<D, false, false>(p, q, k, v, dO, lse2, delta, dk, dv);
}

template <int D, typename T>
hipError_t launch_pre(const Problem& p, const void* o, const void* dO, const float* lse, float* delta, float* lse2) {
  const int64_t rows = (int64_t)p.B * p.H * p.N;
  constexpr int rows_per_block = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D, T>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(256), 0, p.stream, (const T*)o, (const T*)dO, lse, delta, lse2, rows);
  return hipGetLastError();
}

}  // namespace

int64_t bwd_dkdv_bf16_grid(int B, int H, int N) { return (int64_t)((N + kBwdBc - 1) / kBwdBc) * B * H; }

hipError_t launch_bwd_prepare(const Problem& p, bool bf16, const void* o, const void* dO, const float* lse,
                              void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, bf16);
  float* delta = (float*)((char*)workspace + ws.delta_off);
  if (bf16) {
    float* lse2 = (float*)((char*)workspace + ws.lse2_off);
    return p.d == 64 ? launch_pre<64, __bf16>(p, o, dO, lse, delta, lse2)
                     : launch_pre<128, __bf16>(p, o, dO, lse, delta, lse2);
  }
  return p.d == 64 ? launch_pre<64, float>(p, o, dO, lse, delta, nullptr)
                   : launch_pre<128, float>(p, o, dO, lse, delta, nullptr);
}

hipError_t launch_bwd_dkdv_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                                void* dk, void* dv, const void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, true);
  const float* delta = (const float*)((const char*)workspace + ws.delta_off);
  const float* lse2 = (const float*)((const char*)workspace + ws.lse2_off);
#ifndef FA_DKDV_KL
#define FA_DKDV_KL 1
#endif
  if (FA_DKDV_KL && p.d == 128 && p.block_mask == nullptr)
    return launch_dkdv_kl_bf16(p, q, k, v, dO, lse2, delta, dk, dv);
  return p.d == 64 ? launch_dkdv_d<64>(p, q, k, v, dO, lse2, delta, dk, dv)
                   : launch_dkdv_d<128>(p, q, k, v, dO, lse2, delta, dk, dv);
}

}  // namespace fa
