// Forward of exact attention, bf16 inputs, fp32 accumulation, on gfx950 matrix cores.
//
// The method: tile Q, K and V into on-chip blocks; for each block of queries, walk the blocks of
// keys/values, compute that block of scores on chip and fold it into the output with an online
// softmax that carries a running maximum m and normaliser l per row, rescaling the partial output
// when the maximum grows.  The N x N score matrix never reaches HBM and the result is exact
// (aicassindra FlashAttention architecture page, "End-to-end flow"; promptingindex page,
// "Tiling: keeping computation inside SRAM"; NOTE-005: FlashAttention, "Method" and "Key
// components").  The row statistic kept for the backward is LSE = m + ln l (NOTE-005, "Method").
//
// gfx950 design (the pages' A100 tile rule B_c = ceil(M/4d), B_r = min(B_c, d) is not used; the
// tile is set by the register file, LDS and issue model of a CDNA4 compute unit):
//   * one workgroup = 4 waves of one (batch, head), one wave per SIMD; a wave owns 32 query rows
//     (128 per workgroup), fits in 256 registers, and two workgroups share a compute unit so each
//     covers the other's memory and barrier stalls (64 rows per wave is a compile-time option);
//   * Q of the wave stays in registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16);
//     each lane holds one query column of the score tile, so the row max/sum are in-lane (the two
//     lane halves hold different keys of the same queries and are combined once, at the end);
//   * K and V tiles of 64 keys stream through two double-buffered LDS rings with direct
//     buffer->LDS 16-byte loads (rows past N read as zeros); K runs one tile ahead of V, so each load has a full iteration to
//     land before it is read;
//   * software pipeline: S(t+1) = K(t+1) Q^T is issued on the matrix cores while the VALU turns
//     S(t) into P(t) (exp2, bf16 pack, row sums) and O^T += V(t-1)^T P(t-1)^T runs beside it; the
//     instruction streams are interleaved by explicit schedule groups, LDS fragments are read two
//     MFMA steps ahead, and V^T is read through ds_read_b64_tr_b16;
//   * lazy rescaling: the running maximum is only raised when a tile's maximum exceeds it by more
//     than 2^8 (base 2), so p <= 2^8 and the output/normaliser, which share the stale maximum, stay
//     exact; the O rescale (128 accumulator registers) therefore runs a few times per row instead of
//     once per tile.  Normalisation by l is deferred to the epilogue;
//   * masked tiles (causal diagonal, key padding, ragged tail) take a separate exact path;
//   * workgroups are ordered heaviest first (causal) and, when B*H is a multiple of 8, all query
//     blocks of one head go to one XCD (workgroup ids are dealt round-robin over the 8 XCDs), so a
//     head's K/V stays in that XCD's L2.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kFwdWaves = 4;
// Query rows per wave.  32: a wave fits in 256 registers and two workgroups share a compute unit,
// each covering the other's memory and barrier stalls.  64: one workgroup per compute unit, and
// every K/V fragment read from LDS feeds twice as many rows.
constexpr int kFwdRowsPerWave = FA_FWD_ROWS_PER_WAVE;
constexpr int kFwdBr = kFwdWaves * kFwdRowsPerWave;  // query rows per workgroup
constexpr int kFwdBc = 64;                           // keys per tile
constexpr float kLazyRescale = 8.0f;                 // base-2 headroom before the maximum is raised

template <int D, bool CAUSAL, bool PADDED, bool NEG>
__global__ __launch_bounds__(256, kFwdRowsPerWave == 32 ? 2 : 1) void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                          float* __restrict__ LSE, int H, int N, float c_log2,
                                                          const int32_t* __restrict__ seqlens, int nqb, int BH) {
  constexpr int CH = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = kFwdBc * D * 2;      // bytes of one K or V tile
  constexpr int LOADS = kFwdBc * CH / 256;  // 16-byte loads per thread per tile
  constexpr int DS = D / 16;                // k-steps of S = K Q^T
  constexpr int DT = D / 32;                // 32-wide d tiles of O^T
  constexpr int QT = kFwdRowsPerWave / 32;  // 32-row query halves of a wave
  constexpr bool QLDS = D == 128 && QT == 2;  // Q fragments from LDS instead of registers
  constexpr int VALU3 = QT * 4 * 24;        // VALU instructions of P(t): 4 QT groups x (8 fma, 8 exp, 4 cvt, 4 dot)
  // Separate LDS arrays, each referenced statically, so the compiler sees that a direct load into
  // one buffer never aliases the reads of another.
  __shared__ __attribute__((aligned(1024))) char kbuf0_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char qbuf_raw[QLDS ? kFwdWaves * kFwdRowsPerWave * D * 2 : 16];
  FA_LDS char* kbuf0 = (FA_LDS char*)kbuf0_raw;
  FA_LDS char* kbuf1 = (FA_LDS char*)kbuf1_raw;
  FA_LDS char* vbuf0 = (FA_LDS char*)vbuf0_raw;
  FA_LDS char* vbuf1 = (FA_LDS char*)vbuf1_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- work item: (query block, batch*head), heaviest first, XCD-local heads
  const int wid = blockIdx.x;
  int rank, bh;
  if ((BH & 7) == 0) {
    const int hpx = BH >> 3;
    const int j = wid >> 3;
    rank = j / hpx;
    bh = (wid & 7) + 8 * (j - rank * hpx);
  } else {
    rank = wid / BH;
    bh = wid - rank * BH;
  }
  const int qblock = CAUSAL ? (nqb - 1 - rank) : rank;
  const int b = bh / H;
  const int64_t row0 = (int64_t)bh * N;
  const __bf16* Qh = Q + row0 * D;
  const __bf16* Kh = K + row0 * D;
  const __bf16* Vh = V + row0 * D;

  const int L = PADDED ? clamp_len(seqlens, b, N) : N;  // keys >= L are invisible
  const int q0 = qblock * kFwdBr;
  const int qw = q0 + wave * kFwdRowsPerWave;
  const int kv_end = CAUSAL ? min(L, q0 + kFwdBr) : L;
  const int ntiles = (kv_end + kFwdBc - 1) / kFwdBc;  // tiles the workgroup loads
  const int wave_end = CAUSAL ? min(L, qw + kFwdRowsPerWave) : L;
  const int n_wave = (wave_end + kFwdBc - 1) / kFwdBc;  // tiles this wave computes
  int n_full = L / kFwdBc;                              // leading tiles with no hidden pair
  if (CAUSAL) n_full = min(n_full, qw / kFwdBc);

  // Q^T fragments (B operand of S^T = K Q^T): lane holds query qw + 32 qt + l32, d = 16 ds + 8 half
  // .. +7.  d=64: kept in registers.  d=128: the wave's 64 rows are staged once in its own LDS
  // region (16 KiB) and the fragments are read per k-step, which keeps the wave within 256 VGPRs.
  bf16x8 qf[QT][QLDS ? 1 : DS];
  FA_LDS char* qbuf = (FA_LDS char*)qbuf_raw + wave * (QLDS ? kFwdRowsPerWave * D * 2 : 0);
  if constexpr (QLDS) {
    const u32x4 rq = make_rsrc(Qh + (int64_t)qw * D, (N - qw) * D * 2);  // rows past N read as zeros
#pragma unroll
    for (int n = 0; n < kFwdRowsPerWave * CH / 64; ++n) {
      const int p = n * 64 + lane;
      const int r = p / CH;
      const int c = (p % CH) ^ swz<D>(r);
      bload_lds16(rq, (uint32_t)(r * D + 8 * c) * 2, qbuf + n * 1024);
    }
  } else {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
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
  }

  f32x16 acc[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[qt][dt] = zero16();
  float m_run[QT], l_run[QT];  // base-2 running maximum (identical in both lane halves); per-lane
#pragma unroll                 // partial normaliser (this lane's keys)
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }

  // K/V tile loads: buffer loads straight into LDS; rows past N read as zeros (the buffer ends at
  // the head's last row; those keys are masked).  K and V tiles share the per-lane byte offsets,
  // which are loop-invariant.
  uint32_t voff[LOADS];
#pragma unroll
  for (int n = 0; n < LOADS; ++n) {
    const int p = (n * kFwdWaves + wave) * 64 + lane;
    const int r = p / CH;
    const int c = (p % CH) ^ swz<D>(r);
    voff[n] = (uint32_t)(r * D + 8 * c) * 2;
  }
  auto load_tile = [&](const __bf16* src, int t, FA_LDS char* dst) {
    const u32x4 rs = make_rsrc(src + (int64_t)t * kFwdBc * D, (N - t * kFwdBc) * D * 2);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) bload_lds16(rs, voff[n], dst + (n * kFwdWaves + wave) * 1024);
  };

  // S^T(tile in kb) = K Q^T, 4 independent accumulators, one K fragment per (ds, kt)
  auto scores = [&](const FA_LDS char* kb, f32x16 (&s)[2][QT]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[kt][qt] = zero16();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      bf16x8 qd[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        qd[qt] = QLDS ? lds_read_b128(qbuf, tile_off<D>(32 * qt + l32, 16 * ds + 8 * half)) : qf[qt][QLDS ? 0 : ds];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kf = lds_read_b128(kb, tile_off<D>(32 * kt + l32, 16 * ds + 8 * half));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[kt][qt] = mfma32x32x16(kf, qd[qt], s[kt][qt]);
      }
    }
    pipe_schedule<DS, QLDS ? 4 : 2, 2 * QT, 0, 2, 1>();  // fragment reads two k-steps ahead of their MFMAs
  };

  f32x16 s[2][QT];  // S^T(t): s[kt][qt], lane = query column, rows = keys 32 kt + 8 (r/4) + 4 half + r%4
  bf16x8 pf[QT][4], pn[QT][4];  // P(t-1) (consumed by O += P V) and P(t) (being produced), packed bf16
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  const int g = lane >> 4, j = lane & 15;
  const int vrow = 4 * (g >> 1) + (j >> 2);

  // P(t) = exp2(s cf - m) packed to bf16 (the B operand of O^T += V^T P^T), with the row sums taken
  // by v_dot2_f32_bf16 on the packed values, so the normaliser sums exactly the weights used.
  auto probs = [&](float cf, const float (&m_use)[QT]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kt = ks >> 1, base = 8 * (ks & 1);
        bf16x2 pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2 two = {fast_exp2(fmaf(s[kt][qt][base + 2 * e], cf, -m_use[qt])),
                             fast_exp2(fmaf(s[kt][qt][base + 2 * e + 1], cf, -m_use[qt]))};
          pk[e] = __builtin_convertvector(two, bf16x2);
          l_run[qt] = __builtin_amdgcn_fdot2_f32_bf16(pk[e], ones, l_run[qt], false);
        }
        pn[qt][ks] = cat(__builtin_shufflevector(pk[0], pk[1], 0, 1, 2, 3),
                         __builtin_shufflevector(pk[2], pk[3], 0, 1, 2, 3));
      }
  };

  // O^T += V^T P^T for the tile in vb, over 4 k-steps of 16 keys.  V^T fragment for (dt, ks): lane
  // (d = 32 dt + l32, half) needs keys 16 ks + 4 half + 0..3 and 16 ks + 8 + 4 half + 0..3, the key
  // order of pf; two transposing reads supply them.  Each lane reads from two base addresses (rows
  // vrow and vrow + 8) plus compile-time offsets of 16 rows.
  auto pv = [&](const FA_LDS char* vb) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      // rows vrow + 16 ks share the swizzle; rows vrow + 8 + 16 ks need their own base
      const uint32_t off0 = tile_off<D>(vrow, 32 * dt + 16 * (g & 1) + 4 * (j & 3));
      const uint32_t off8 = tile_off<D>(vrow + 8, 32 * dt + 16 * (g & 1) + 4 * (j & 3));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 vf = cat(lds_read_tr(vb, off0 + ks * 16 * D * 2), lds_read_tr(vb, off8 + ks * 16 * D * 2));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) acc[qt][dt] = mfma32x32x16(vf, pf[qt][ks], acc[qt][dt]);
      }
    }
  };

  if (ntiles > 0) {
    load_tile(Kh, 0, kbuf0);
    if (ntiles > 1) load_tile(Kh, 1, kbuf1);
  }
  // The first iteration adds P(-1) V(-1) with P(-1) = 0 from a zeroed buffer: an exact no-op that
  // keeps a single (interleaved) code path for every iteration.
  for (int i = threadIdx.x; i < TILE / 16; i += 256) *(FA_LDS u32x4*)(vbuf1 + 16 * i) = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[qt][ks][e] = (__bf16)0.f;
  wait_vmem();
  __syncthreads();
  if (n_wave > 0) scores(kbuf0, s);

  // Iteration t (0 <= t <= ntiles): S(t) is in s and P(t-1) in pf.  kn holds K(t+1), vp holds V(t-1);
  // K(t+2) is loaded into kl and V(t) into vl (both last read in iteration t-1).  Every wave runs
  // all ntiles + 1 iterations (one barrier each) in one of four forms, chosen outside the loop so
  // that each form is straight-line code (a data-dependent branch around in-place updates of the
  // score registers makes the compiler copy them on every iteration):
  //   kClean  (t < n_clean):           lazy maximum check; [O += P(t-1) V(t-1) || P(t)]; S(t+1)
  //   kMasked (n_clean <= t < n_wave): mask + exact maximum update; the same products
  //   kDrain  (t == n_wave):           O += P(t-1) V(t-1) only
  //   kIdle   (t > n_wave):            only the workgroup's loads
  // (S(t+1) is computed even when no tile t+1 follows; it is then unused.)
  constexpr int kClean = 0, kMasked = 1, kDrain = 2, kIdle = 3;
  auto step = [&](auto mode, int t, const FA_LDS char* kn, FA_LDS char* kl, const FA_LDS char* vp, FA_LDS char* vl)
      __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode)::value;
    wait_vmem();  // K(t+1) and V(t-1), issued one iteration ago, have landed
    barrier();
    if (t + 2 < ntiles) load_tile(Kh, t + 2, kl);
    if (t < ntiles) load_tile(Vh, t, vl);
    if constexpr (MODE == kDrain) pv(vp);
    if constexpr (MODE == kClean || MODE == kMasked) {
      // ---- prepare: the lazy maximum check (fully visible tile) or mask + exact update
      float cf, m_use[QT], alpha[QT];
      bool raise;
      if constexpr (MODE == kClean) {
        float tm[QT];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          float e = s[0][qt][0];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = (kt == 0 ? 1 : 0); r < 16; ++r) e = NEG ? fminf(e, s[kt][qt][r]) : fmaxf(e, s[kt][qt][r]);
          e = NEG ? min_halves(e) : max_halves(e);
          tm[qt] = e * c_log2;
          alpha[qt] = 1.f;
        }
        bool over = false;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) over |= tm[qt] > m_run[qt] + kLazyRescale;
        raise = __builtin_amdgcn_readfirstlane(__any(over));
        if (raise) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            const float m_new = fmaxf(m_run[qt], tm[qt]);
            alpha[qt] = fast_exp2(m_run[qt] - m_new);
            m_run[qt] = m_new;
          }
        }
        cf = c_log2;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) m_use[qt] = m_run[qt];
      } else {
        const int key0 = t * kFwdBc;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int query = qw + 32 * qt + l32;
          float mx = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
              const bool vis = (key < L) & (!CAUSAL | (key <= query));
              const float v = vis ? s[kt][qt][r] * c_log2 : -INFINITY;
              s[kt][qt][r] = v;
              mx = fmaxf(mx, v);
            }
          mx = max_halves(mx);
          const float m_new = fmaxf(m_run[qt], mx);
          m_use[qt] = (m_new == -INFINITY) ? 0.f : m_new;
          alpha[qt] = fast_exp2(m_run[qt] - m_use[qt]);
          m_run[qt] = m_new;
        }
        cf = 1.f;
        bool changed = false;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) changed |= alpha[qt] != 1.f;
        raise = __builtin_amdgcn_readfirstlane(__any(changed));
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) l_run[qt] *= alpha[qt];
      __builtin_amdgcn_sched_barrier(0);

      // ---- O += P(t-1) V(t-1) on the matrix cores, interleaved with P(t) on the VALU
      probs(cf, m_use);
      pv(vp);
      // 4 DT steps of (2 transposing reads -> 2 MFMAs), each MFMA followed by its share of the VALU work
      pipe_schedule<4 * DT, 2, QT, VALU3 / (4 * DT * QT), 2, 0>();
      // Pin P(t) and the row sums here: without a use inside this phase the compiler sinks their
      // computation past the matrix-core work it is meant to overlap.
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(pn[qt][ks]));
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) asm volatile("" : "+v"(l_run[qt]));
      __builtin_amdgcn_sched_barrier(0);
      if (raise) {  // O carries P(t-1) at the old maximum: scale it to the new one
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[qt][dt] *= alpha[qt];
      }
      // ---- S(t+1) = K(t+1) Q^T
      scores(kn, s);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) pf[qt][ks] = pn[qt][ks];
    }
  };
  // even t: K(t+1) in kbuf1, K(t+2) -> kbuf0, V(t-1) in vbuf1, V(t) -> vbuf0; odd t: the other way
  // round.  Outside the unrolled clean loop the buffers are picked at run time (one copy of each
  // form; two copies of the masked form would not fit the register budget).
  auto at = [&](auto mode, int t) __attribute__((always_inline)) {
    const bool odd = t & 1;
    step(mode, t, odd ? kbuf0 : kbuf1, odd ? kbuf1 : kbuf0, odd ? vbuf0 : vbuf1, odd ? vbuf1 : vbuf0);
  };
  using Clean = std::integral_constant<int, kClean>;
  const int n_clean = min(n_full, n_wave);
  int t = 0;
  for (; t + 1 < n_clean; t += 2) {
    step(Clean{}, t, kbuf1, kbuf0, vbuf1, vbuf0);
    step(Clean{}, t + 1, kbuf0, kbuf1, vbuf0, vbuf1);
  }
  if (t < n_clean) step(Clean{}, t++, kbuf1, kbuf0, vbuf1, vbuf0);
  for (; t < n_wave; ++t) at(std::integral_constant<int, kMasked>{}, t);
  at(std::integral_constant<int, kDrain>{}, t++);  // t == n_wave <= ntiles
  for (; t <= ntiles; ++t) at(std::integral_constant<int, kIdle>{}, t);

  // ---- epilogue: O = acc / l (bf16, RNE); LSE = (m + log2 l) ln 2
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int query = qw + 32 * qt + l32;
    const float l = add_halves(l_run[qt]);
    const bool has = l > 0.f;
    const float inv = has ? 1.f / l : 0.f;
    if (query < N) {
      if (half == 0) LSE[row0 + query] = has ? (m_run[qt] + __log2f(l)) * kLn2 : -INFINITY;
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

template <int D, bool CAUSAL, bool PADDED, bool NEG>
hipError_t launch(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  const int nqb = (p.N + kFwdBr - 1) / kFwdBr;
  const int BH = p.B * p.H;
  const float c_log2 = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, PADDED, NEG>), dim3((unsigned)(nqb * BH)), dim3(256), 0, p.stream,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, p.H, p.N, c_log2,
                     p.seqlens, nqb, BH);
  return hipGetLastError();
}

template <int D, bool NEG>
hipError_t launch_mask(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  const bool pad = p.seqlens != nullptr;
  if (p.causal)
    return pad ? launch<D, true, true, NEG>(p, q, k, v, o, lse) : launch<D, true, false, NEG>(p, q, k, v, o, lse);
  return pad ? launch<D, false, true, NEG>(p, q, k, v, o, lse) : launch<D, false, false, NEG>(p, q, k, v, o, lse);
}

template <int D>
hipError_t launch_d(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  return p.scale < 0.f ? launch_mask<D, true>(p, q, k, v, o, lse) : launch_mask<D, false>(p, q, k, v, o, lse);
}

}  // namespace

int64_t fwd_bf16_grid(int B, int H, int N) { return (int64_t)((N + kFwdBr - 1) / kFwdBr) * B * H; }

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  return p.d == 64 ? launch_d<64>(p, q, k, v, o, lse) : launch_d<128>(p, q, k, v, o, lse);
}

}  // namespace fa
