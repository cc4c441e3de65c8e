// Forward of exact attention, bf16 inputs, fp32 accumulation, on gfx950 matrix cores.
//
// The method: tile Q, K and V into on-chip blocks; for each block of queries, walk the blocks of
// keys/values, compute that block of scores on chip and fold it into the output with an online
// softmax that carries a running maximum m and normaliser l per row, rescaling the partial output
// whenever the maximum grows.  The N x N score matrix never reaches HBM, and the result is exact.
// (aicassindra FlashAttention architecture page, "End-to-end flow"; promptingindex page,
// "Tiling: keeping computation inside SRAM"; NOTE-005: FlashAttention, "Method" and "Key
// components").  The row statistic kept for the backward is LSE = m + ln l (NOTE-005, "Method").
//
// gfx950 design (the pages' A100 tile rule B_c = ceil(M/4d), B_r = min(B_c, d) is not used; the
// tile is set by LDS bandwidth and register capacity of a CDNA4 compute unit):
//   * one workgroup = 4 waves = 256 query rows of one (batch, head); each wave owns 64 rows,
//     so every K/V byte read from LDS feeds 64 query rows (LDS traffic is half the MFMA rate);
//   * Q of the wave stays in registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16),
//     so each lane holds one query column of the score tile and the row reductions of the
//     softmax are in-lane plus one v_permlane32_swap;
//   * K and V tiles of 64 keys stream through a double-buffered LDS ring with direct
//     global->LDS 16-byte loads, prefetching tile t+1 while tile t is computed;
//   * P^T goes from the accumulator registers straight into the B operand of O^T += V^T P^T
//     (the key order inside each 16-key MFMA step is permuted consistently on both operands);
//     V^T comes from LDS through the transposing read ds_read_b64_tr_b16;
//   * the softmax works in base 2 with scale*log2(e) folded into one FMA before v_exp_f32, and
//     normalisation by l is deferred to the epilogue;
//   * causal: query blocks are launched heaviest first; a wave skips key tiles past its diagonal.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kFwdWaves = 4;
constexpr int kFwdRowsPerWave = 64;
constexpr int kFwdBr = kFwdWaves * kFwdRowsPerWave;  // 256 query rows per workgroup
constexpr int kFwdBc = 64;                           // keys per tile

template <int D, bool CAUSAL, bool PADDED>
__global__ __launch_bounds__(256, 1) void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                          float* __restrict__ LSE, int H, int N, float c_log2,
                                                          const int32_t* __restrict__ seqlens, int num_qblocks) {
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int TILE = kFwdBc * D * 2;        // bytes of one K or V tile
  constexpr int LOADS = kFwdBc * CH / 256;    // 16-byte loads per thread per tile
  constexpr int DS = D / 16;                  // k-steps of S = K Q^T
  constexpr int DT = D / 32;                  // 32-wide d tiles of O^T
  // Two separate LDS arrays (not one indexed ring) so the compiler can see that the prefetch into
  // one buffer never aliases the reads of the other and does not wait for it.
  __shared__ __attribute__((aligned(1024))) char buf0_raw[2 * TILE];  // K | V
  __shared__ __attribute__((aligned(1024))) char buf1_raw[2 * TILE];
  FA_LDS char* buf0 = (FA_LDS char*)buf0_raw;
  FA_LDS char* buf1 = (FA_LDS char*)buf1_raw;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int qblock = CAUSAL ? (num_qblocks - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t row0 = ((int64_t)b * H + h) * N;
  const __bf16* Qh = Q + row0 * D;
  const __bf16* Kh = K + row0 * D;
  const __bf16* Vh = V + row0 * D;

  const int L = PADDED ? clamp_len(seqlens, b, N) : N;  // keys >= L are invisible
  const int q0 = qblock * kFwdBr;
  const int qw = q0 + wave * kFwdRowsPerWave;
  int kv_end = L;
  if (CAUSAL) kv_end = min(kv_end, q0 + kFwdBr);
  const int ntiles = (kv_end + kFwdBc - 1) / kFwdBc;
  int wave_end = kv_end;
  if (CAUSAL) wave_end = min(kv_end, qw + kFwdRowsPerWave);
  const int wave_tiles = wave_end > 0 ? (wave_end + kFwdBc - 1) / kFwdBc : 0;

  // Q^T fragments (B operand): lane holds query qw + 32 qt + l32, d = 16 ds + 8 half .. +7.
  bf16x8 qf[2][DS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int row = qw + 32 * qt + l32;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      if (row < N) {
        qf[qt][ds] = *(const bf16x8*)(Qh + (int64_t)row * D + 16 * ds + 8 * half);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qt][ds][e] = (__bf16)0.f;
      }
    }
  }

  f32x16 acc[2][DT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[qt][dt] = zero16();
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  auto issue_tile = [&](int t, FA_LDS char* kdst) {
    FA_LDS char* vdst = kdst + TILE;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int slot = (n * kFwdWaves + wave) * 64;  // first 16-byte slot of this wave's 1 KiB
      const int p = slot + lane;
      const int r = p / CH;
      const int c = (p % CH) ^ swz(r);
      const int key = min(t * kFwdBc + r, N - 1);  // rows past N are masked; read a valid row
      gload_lds16(Kh + (int64_t)key * D + 8 * c, kdst + slot * 16);
      gload_lds16(Vh + (int64_t)key * D + 8 * c, vdst + slot * 16);
    }
  };

  // One step: wait for tile t in `cur`, start tile t+1 into `nxt`, then compute tile t.
  auto step = [&](int t, const FA_LDS char* cur, FA_LDS char* nxt) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < ntiles) issue_tile(t + 1, nxt);
    if (t < wave_tiles) {
      const FA_LDS char* kb = cur;
      const FA_LDS char* vb = cur + TILE;
      // ---- S^T = K Q^T for 64 keys x 64 queries: s[kt][qt]
      f32x16 s[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) s[kt][qt] = zero16();
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bf16x8 kf = lds_read_b128(kb, tile_off<D>(32 * kt + l32, 16 * ds + 8 * half));
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) s[kt][qt] = mfma32x32x16(kf, qf[qt][ds], s[kt][qt]);
        }
      }
      // ---- mask (only tiles that reach past L or the wave's diagonal).  A masked tile is moved to
      // the scaled domain t = s * scale * log2(e) first, with -inf for hidden pairs, so the update
      // below runs with a unit factor (a hidden pair never meets a zero or negative scale).
      const int key0 = t * kFwdBc;
      const bool need_mask = (key0 + kFwdBc > L) || (CAUSAL && key0 + kFwdBc - 1 > qw);
      float cf = c_log2;
      if (need_mask) {
        cf = 1.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            const int query = qw + 32 * qt + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
              const bool vis = key < L && (!CAUSAL || key <= query);
              s[kt][qt][r] = vis ? s[kt][qt][r] * c_log2 : -INFINITY;
            }
          }
      }
      // ---- online softmax (base 2): m, l per query column; rescale O^T columns by alpha
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float ext;
        if (cf >= 0.f) {
          float mx = s[0][qt][0];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][qt][r]);
          ext = max_halves(mx);
        } else {
          float mn = s[0][qt][0];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mn = fminf(mn, s[kt][qt][r]);
          ext = min_halves(mn);
        }
        const float tile_max = (ext == -INFINITY) ? -INFINITY : ext * cf;
        const float m_new = fmaxf(m_run[qt], tile_max);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[qt] - m_use);
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(s[kt][qt][r], cf, -m_use));
            s[kt][qt][r] = p;
            rs += p;
          }
        rs = add_halves(rs);
        l_run[qt] = l_run[qt] * alpha + rs;
        m_run[qt] = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[qt][dt] *= alpha;
      }
      // ---- O^T += V^T P^T over 4 k-steps of 16 keys
      bf16x8 pf[2][4];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) pf[qt][ks] = pack8(s[ks >> 1][qt], 8 * (ks & 1));
      // V^T fragment for (dt, ks): lane (d = 32 dt + l32, half) needs keys 16 ks + 4 half + 0..3 and
      // 16 ks + 8 + 4 half + 0..3, the same key order as pf.  Two transposing reads supply them.
      // Rows 16 ks + r and 16 ks + 8 + r share the swizzle, so every read of a lane is one base
      // address plus a compile-time offset.
      const int g = lane >> 4, j = lane & 15;
      const int vrow = 4 * (g >> 1) + (j >> 2);
      u32x2 vfr[2][4][2];
      auto read_v = [&](u32x2 (&dst)[4][2], int dt) {
        const uint32_t base = lds_addr(vb) + tile_off<D>(vrow, 32 * dt + 16 * (g & 1) + 4 * (j & 3));
        dst[0][0] = lds_read_tr_asm<0 * 16 * D * 2>(base);
        dst[0][1] = lds_read_tr_asm<(0 * 16 + 8) * D * 2>(base);
        dst[1][0] = lds_read_tr_asm<1 * 16 * D * 2>(base);
        dst[1][1] = lds_read_tr_asm<(1 * 16 + 8) * D * 2>(base);
        dst[2][0] = lds_read_tr_asm<2 * 16 * D * 2>(base);
        dst[2][1] = lds_read_tr_asm<(2 * 16 + 8) * D * 2>(base);
        dst[3][0] = lds_read_tr_asm<3 * 16 * D * 2>(base);
        dst[3][1] = lds_read_tr_asm<(3 * 16 + 8) * D * 2>(base);
      };
      read_v(vfr[0], 0);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        u32x2 (&cur)[4][2] = vfr[dt & 1];
        lds_wait(cur[0][0], cur[0][1], cur[1][0], cur[1][1], cur[2][0], cur[2][1], cur[3][0], cur[3][1]);
        if (dt + 1 < DT) read_v(vfr[(dt + 1) & 1], dt + 1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 vf = cat(cur[ks][0], cur[ks][1]);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) acc[qt][dt] = mfma32x32x16(vf, pf[qt][ks], acc[qt][dt]);
        }
      }
    }
  };

  if (ntiles > 0) issue_tile(0, buf0);
  for (int t = 0; t < ntiles; t += 2) {
    step(t, buf0, buf1);
    if (t + 1 < ntiles) step(t + 1, buf1, buf0);
  }

  // ---- epilogue: O = acc / l (bf16, RNE); LSE = (m + log2 l) ln 2
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int query = qw + 32 * qt + l32;
    const bool has = l_run[qt] > 0.f;
    const float inv = has ? 1.f / l_run[qt] : 0.f;
    if (query < N) {
      if (half == 0) LSE[row0 + query] = has ? (m_run[qt] + __log2f(l_run[qt])) * kLn2 : -INFINITY;
      __bf16* orow = O + (row0 + query) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d0 = 32 * dt + 8 * gq + 4 * half;
          const bf16x4 v4 = pack4(acc[qt][dt][4 * gq] * inv, acc[qt][dt][4 * gq + 1] * inv,
                                  acc[qt][dt][4 * gq + 2] * inv, acc[qt][dt][4 * gq + 3] * inv);
          *(bf16x4*)(orow + d0) = v4;
        }
    }
  }
}

template <int D, bool CAUSAL, bool PADDED>
hipError_t launch(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  const int nqb = (p.N + kFwdBr - 1) / kFwdBr;
  dim3 grid(nqb, p.H, p.B);
  const float c_log2 = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, PADDED>), grid, dim3(256), 0, p.stream, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, p.H, p.N, c_log2, p.seqlens, nqb);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  const bool pad = p.seqlens != nullptr;
  if (p.causal) return pad ? launch<D, true, true>(p, q, k, v, o, lse) : launch<D, true, false>(p, q, k, v, o, lse);
  return pad ? launch<D, false, true>(p, q, k, v, o, lse) : launch<D, false, false>(p, q, k, v, o, lse);
}

}  // namespace

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  return p.d == 64 ? launch_d<64>(p, q, k, v, o, lse) : launch_d<128>(p, q, k, v, o, lse);
}

}  // namespace fa
