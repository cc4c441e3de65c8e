// dQ of the backward of exact attention, bf16 inputs, fp32 accumulation, on gfx950 matrix cores.
//
// dQ = scale dS K with dS = P * (dP - D), P = exp(S - LSE), S = scale Q K^T, dP = dO V^T: the
// probabilities are recomputed block by block from the stored per-row log-sum-exp, never read
// from a stored N x N matrix (NOTE-005: FlashAttention, "Method").  This kernel walks the key
// blocks of a block of queries, like the forward, and writes dQ once, so no two workgroups ever
// add into the same dQ row: dK and dV come from the key-block-outer kernel (fa_bwd_bf16.hip),
// which therefore needs no atomic additions.  (Float atomics execute at the memory side on this
// GPU at roughly 300 G operations/s; accumulating dQ that way made the backward bound by them.)
//
// gfx950 design (shared with the forward kernel):
//   * one workgroup = 8 waves = 256 query rows of one (batch, head), one workgroup per compute unit;
//     a wave owns 32 rows and fits in 256 registers, so two waves share each SIMD and cover each
//     other's stalls (a build with FA_DQ_WAVES=4 makes 128-row workgroups, two per compute unit);
//   * Q^T and dO^T of the wave stay in registers as B operands of S^T = K Q^T and dP^T = V dO^T
//     (v_mfma_f32_32x32x16_bf16); each lane holds one query column, so LSE and D are one scalar
//     per lane;
//   * K and V tiles of 64 keys pass through an LDS ring filled by direct buffer->LDS loads: at
//     d = 128 three stages fetched two tiles ahead, one barrier per tile; at d = 64 four stages
//     filled two tiles at a time, one barrier per two tiles (the 4-wave build: two stages).  K is
//     read twice: row-major for S^T and through the transposing read for dQ^T += K^T dS^T;
//   * dS^T goes from registers straight into the B operand of the dQ^T product (the key order
//     inside each 16-key step is permuted the same way on both operands);
//   * tiles with hidden pairs (causal diagonal, key padding, ragged tail) set the hidden scores to
//     -inf first; workgroups are ordered heaviest first and, when B*H is a multiple of 8, all
//     query blocks of one head go to one XCD.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

#ifndef FA_DQ_WAVES
#define FA_DQ_WAVES 8
#endif
// 8 waves (two per SIMD) share each K/V tile and one workgroup occupies a compute unit; 4 waves use
// two stages and two workgroups per compute unit.
constexpr int kDqWaves = FA_DQ_WAVES;
// Tiles per barrier.  d = 64 (8 waves): two, through a four-stage ring (two tiles loaded after each
// barrier, the waves meet once per two tiles; measured -1 to -4 % dQ time at d = 64).  d = 128: one,
// through a three-stage ring fetched two tiles ahead (the grouped loop spills there).
template <int D>
constexpr int dq_group() { return kDqWaves == 8 && D == 64 ? 2 : 1; }
template <int D>
constexpr int dq_stages() { return dq_group<D>() > 1 ? 2 * dq_group<D>() : (kDqWaves == 8 ? 3 : 2); }
constexpr int kDqRowsPerWave = 32;
constexpr int kDqBr = kDqWaves * kDqRowsPerWave;  // query rows per workgroup
constexpr int kDqBc = 64;                         // keys per tile

template <int D, bool CAUSAL, bool PADDED, bool SPARSE, bool DROP>
__global__ __launch_bounds__(kDqWaves * 64, kDqWaves == 8 ? 1 : 2) void bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                        const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                        float* __restrict__ LSE2, float* __restrict__ DELTA,
                                                        __bf16* __restrict__ dQ, const __bf16* __restrict__ Opre,
                                                        const float* __restrict__ LSEpre,
                                                        int H, int N, float scale, float c_log2,
                                                        const int32_t* __restrict__ seqlens,
                                                        const uint8_t* __restrict__ bmask, Dropout dr, int nqb,
                                                        int BH) {
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int TILE = kDqBc * D * 2;      // bytes of one K or V tile
  constexpr int LOADS = kDqBc * CH / (64 * kDqWaves);  // 16-byte loads per thread per tile
  constexpr int DS = D / 16;               // k-steps of S^T = K Q^T
  constexpr int DT = D / 32;               // 32-wide d tiles of dQ^T
  // Separate, statically referenced stages (K and V of tile t in stage t % dq_stages<D>())
  __shared__ __attribute__((aligned(1024))) char kbuf0_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf2_raw[dq_stages<D>() > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(1024))) char kbuf3_raw[dq_stages<D>() > 3 ? TILE : 16];
  __shared__ __attribute__((aligned(1024))) char vbuf0_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf2_raw[dq_stages<D>() > 2 ? TILE : 16];
  __shared__ __attribute__((aligned(1024))) char vbuf3_raw[dq_stages<D>() > 3 ? TILE : 16];
  FA_LDS char* const kst[4] = {(FA_LDS char*)kbuf0_raw, (FA_LDS char*)kbuf1_raw, (FA_LDS char*)kbuf2_raw,
                               (FA_LDS char*)kbuf3_raw};
  FA_LDS char* const vst[4] = {(FA_LDS char*)vbuf0_raw, (FA_LDS char*)vbuf1_raw, (FA_LDS char*)vbuf2_raw,
                               (FA_LDS char*)vbuf3_raw};
  // block-sparse: the key tiles visible to any of the workgroup's query blocks, in order, with one
  // flag bit per query block (two tiles per mask block)
  __shared__ uint16_t tlist_raw[SPARSE ? 2 * kMaxMaskBlocks : 1];
  __shared__ int tcount_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // ---- work item: (query block, batch*head), heaviest first, XCD-local heads
  const int wid = work_item();
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
  const __bf16* dOh = dO + row0 * D;

  const int L = PADDED ? clamp_len(seqlens, b, N) : N;  // keys >= L are invisible
  const int q0 = qblock * kDqBr;
  const int qw = q0 + wave * kDqRowsPerWave;
  const int kv_end = CAUSAL ? min(L, q0 + kDqBr) : L;
  int ntiles = (kv_end + kDqBc - 1) / kDqBc;  // tiles the workgroup loads
  const int wave_end = CAUSAL ? min(L, qw + kDqRowsPerWave) : L;
  int n_wave = (wave_end + kDqBc - 1) / kDqBc;  // tiles this wave computes
  int n_full = L / kDqBc;                       // leading tiles with no hidden pair
  if (CAUSAL) n_full = min(n_full, qw / kDqBc);
  // Block-sparse: the steps walk the list of tiles visible to some query block of the workgroup;
  // a wave computes a tile only when its own block's flag is set.  n_wave becomes a list position;
  // n_full stays a tile index (the masking of a tile depends on where it is, not on the list).
  const FA_LDS uint16_t* const tlist = (const FA_LDS uint16_t*)tlist_raw;
  constexpr int kBlocksPerWg = kDqBr / kMaskBlock;
  const int wbit = (wave * kDqRowsPerWave) / kMaskBlock;  // this wave's query block within the workgroup
  if constexpr (SPARSE) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const int qb0 = q0 / kMaskBlock;
    const uint8_t* brow = bmask + ((int64_t)bh * nb + qb0) * nb;
    if (wave == 0)
      compact_tiles<kMaskBlock / kDqBc>((FA_LDS uint16_t*)tlist_raw, (FA_LDS int*)&tcount_raw, 0, (ntiles + 1) / 2,
                                        ntiles, [&](int kb) {
                                          int f = 0;
#pragma unroll
                                          for (int g = 0; g < kBlocksPerWg; ++g)
                                            if (qb0 + g < nb && brow[(int64_t)g * nb + kb] != 0) f |= 1 << g;
                                          return f;
                                        });
    __syncthreads();
    const int n = *(volatile FA_LDS int*)&tcount_raw;
    n_wave = count_below(tlist, n, n_wave);
    ntiles = n;
  }
  auto tix = [&](int t) { return SPARSE ? list_tile(tlist[t]) : t; };
  auto mine = [&](int t) { return !SPARSE || ((list_flags(tlist[t]) >> wbit) & 1); };

  // Q^T and dO^T fragments (B operands): lane holds query qw + l32, d = 16 ds + 8 half .. +7
  const int query = qw + l32;
  const int qrow = min(query, N - 1);
  bf16x8 qf[DS], gf[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    qf[ds] = *(const bf16x8*)(Qh + (int64_t)qrow * D + 16 * ds + 8 * half);
    gf[ds] = *(const bf16x8*)(dOh + (int64_t)qrow * D + 16 * ds + 8 * half);
  }
  float lse2, del;  // LSE log2(e) and D = sum_c dO_c O_c of this lane's query (the workspace holds -D)
  if (Opre == nullptr) {
    lse2 = LSE2[row0 + qrow];
    del = -DELTA[row0 + qrow];
  } else {
    // The prepare stage folded in: D from this lane's dO fragments and the same fragments of O, summed
    // in the prepare kernel's order (8 products per part of 8 columns, part p = 2 ds + half, then a tree
    // over the parts: p ^ 8 .. p ^ 2 in the lane, p ^ 1 across the lane halves), so it is bitwise
    // what that kernel writes; stored for the dK/dV pass with LSE log2(e).
    float sp[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8 of = *(const bf16x8*)(Opre + (row0 + qrow) * D + 16 * ds + 8 * half);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf((float)of[e], (float)gf[ds][e], a);
      sp[ds] = a;
    }
#pragma unroll
    for (int st = DS / 2; st >= 1; st >>= 1) {
      float t[DS];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) t[ds] = sp[ds] + sp[ds ^ st];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) sp[ds] = t[ds];
    }
    del = add_halves(sp[0]);
    lse2 = LSEpre[row0 + qrow] * kLog2e;
    if (half == 0 && query < N) {
      DELTA[row0 + query] = -del;
      LSE2[row0 + query] = lse2;
    }
  }

  // The dP^T accumulators start from -D (this lane's query in all 16 elements, kept in registers for
  // the whole walk), so the matrix cores produce dP - D and dS needs one multiply per score: -3 to
  // -6 % dQ time.  With dropout they start from -D t / 256, so that a kept element's (256 / t) dP - D
  // needs one multiply (and t = 256 gives the dense values bitwise).  Where the 16 registers do not
  // fit beside the rest (d = 128 without the causal mask, which then spills), D is subtracted instead.
  constexpr bool kNdInit = D == 64 || CAUSAL;
  const float ndel0 = DROP ? -del * ((float)dr.t * (1.f / 256.f)) : -del;
  f32x16 ndel16;
  if constexpr (kNdInit && !DROP) {
#pragma unroll
    for (int r = 0; r < 16; ++r) ndel16[r] = ndel0;
  }
  f32x16 acc[DT];  // dQ^T [d][q]: lane = query column, rows d = 32 dt + 8 (r/4) + 4 half + r%4
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();

  // K/V tile loads: buffer loads straight into LDS; rows past N read as zeros (the buffer ends at
  // the head's last row; those keys are masked).  Per-lane byte offsets inside a tile are
  // loop-invariant.
  uint32_t voff[LOADS];
#pragma unroll
  for (int n = 0; n < LOADS; ++n) {
    const int p = (n * kDqWaves + wave) * 64 + lane;
    const int r = p / CH;
    const int c = (p % CH) ^ swz<D>(r);
    voff[n] = (uint32_t)(r * D + 8 * c) * 2;
  }
  // One buffer resource per tensor over the whole head (built once): a tile's byte offset goes into the
  // per-lane offset, which the range check covers, so rows past N still read as zeros.
  const u32x4 rK = make_rsrc(Kh, N * D * 2), rV = make_rsrc(Vh, N * D * 2);
  auto load_tile = [&](const u32x4& rs, int t, FA_LDS char* dst) {
    const uint32_t tb = (uint32_t)tix(t) * kDqBc * D * 2;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) bload_lds16(rs, voff[n] + tb, dst + (n * kDqWaves + wave) * 1024);
  };

  const int g = lane >> 4, j = lane & 15;
  const int trow = 4 * (g >> 1) + (j >> 2);

  // One 32-key half kt of a key tile: S^T, dP^T (MFMA) -> P^T, dS^T (VALU) -> dQ^T += K^T dS^T
  // (MFMA).  The halves run one after the other so that a wave's live state fits the register
  // budget of two waves per SIMD; the other workgroup on the compute unit fills the gaps.
  auto half_tile = [&](int t, int kt, const FA_LDS char* kb, const FA_LDS char* vb) __attribute__((always_inline)) {
    f32x16 s = zero16(), dp = zero16();
    if constexpr (kNdInit) {
      if constexpr (DROP) {
        // rebuilt for every half tile (from a value made opaque, so the splat is not hoisted out of
        // the loop): with the dropout state beside it a persistent copy does not fit in the
        // registers at d = 128
        float x = ndel0;
        asm volatile("" : "+v"(x));
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = x;
      } else {
        dp = ndel16;
      }
    }
    constexpr int RRA = D == 128 ? 1 : 2;  // K/V row fragments read RRA k-steps ahead
    bf16x8 fk[RRA + 1], fv[RRA + 1];
    auto rd = [&](int ds, bf16x8& k, bf16x8& v) {
      const uint32_t off = tile_off<D>(32 * kt + l32, 16 * ds + 8 * half);
      k = lds_read_b128(kb, off);
      v = lds_read_b128(vb, off);
    };
#pragma unroll
    for (int ds = 0; ds < RRA; ++ds) rd(ds, fk[ds], fv[ds]);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      __builtin_amdgcn_sched_barrier(0);
      if (ds + RRA < DS) rd(ds + RRA, fk[(ds + RRA) % (RRA + 1)], fv[(ds + RRA) % (RRA + 1)]);
      s = mfma32x32x16(fk[ds % (RRA + 1)], qf[ds], s);
      dp = mfma32x32x16(fv[ds % (RRA + 1)], gf[ds], dp);
    }
    __builtin_amdgcn_sched_barrier(0);

    // P^T = exp2(S^T c - LSE log2 e), hidden pairs 0; dS^T = P^T (dP^T - D), packed to bf16 in the
    // B-operand key order of the dQ^T product
    float cf = c_log2;
    float sv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = s[r];
    if (t >= n_full) {
      // element r holds key key0 + 8 (r / 4) + 4 half + r % 4, visible iff below this lane's limit
      const int lim = (CAUSAL ? min(L, query + 1) : L) - (t * kDqBc + 32 * kt + 4 * half);
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = (8 * (r >> 2) + (r & 3)) < lim ? sv[r] * c_log2 : -INFINITY;
      cf = 1.f;
    }
    // dropout: dP of the kept elements, scaled by 256/t; the others contribute P (0 - D)
    u32x4 kwd = {};
    if constexpr (DROP) kwd = dropout_words(dr, (uint32_t)bh, query, 2 * t + kt, half);
    bf16x8 dsb[2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      float d8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * kh + e;
        const float p = fast_exp2(fmaf(sv[r], cf, -lse2));
        float dpv = dp[r];
        if constexpr (kNdInit) {  // dpv = dP - D (dropout: dP - D t / 256), accumulated by the matrix cores
          if constexpr (DROP) dpv = dropout_keep(dr, kwd[r >> 2], r & 3) ? dpv * dr.scale : -del;
          d8[e] = p * dpv;
        } else {
          if constexpr (DROP) dpv = dropout_keep(dr, kwd[r >> 2], r & 3) ? dpv * dr.scale : 0.f;
          d8[e] = p * (dpv - del);
        }
      }
      dsb[kh] = pack8f(d8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // dQ^T += K^T dS^T: K^T fragment (lane: d = 32 dt + l32; keys 16 ks + 4 half + 0..3 and
    // 16 ks + 8 + 4 half + 0..3) from two transposing reads (bases for rows trow and trow + 8)
    constexpr int TRA = D == 128 ? 3 : 2;  // K^T fragments read TRA products ahead
    bf16x8 fa[TRA + 1];
    auto rdk = [&](int i, bf16x8& a) {
      const int dt = i >> 1, ks = 2 * kt + (i & 1);
      const uint32_t b0 = tile_off<D>(trow, 32 * dt + 16 * (g & 1) + 4 * (j & 3)) + ks * 16 * D * 2;
      const uint32_t b8 = tile_off<D>(trow + 8, 32 * dt + 16 * (g & 1) + 4 * (j & 3)) + ks * 16 * D * 2;
      a = cat(lds_read_tr(kb, b0), lds_read_tr(kb, b8));
    };
#pragma unroll
    for (int i = 0; i < TRA; ++i) rdk(i, fa[i]);
#pragma unroll
    for (int i = 0; i < 2 * DT; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + TRA < 2 * DT) rdk(i + TRA, fa[(i + TRA) % (TRA + 1)]);
      acc[i >> 1] = mfma32x32x16(fa[i % (TRA + 1)], dsb[i & 1], acc[i >> 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto tile = [&](int t, const FA_LDS char* kb, const FA_LDS char* vb) __attribute__((always_inline)) {
    half_tile(t, 0, kb, vb);
    half_tile(t, 1, kb, vb);
  };

  // Step t: tile t (stage t % NS) must have landed; the next NS - 2 tiles may still be in flight.
  // After the barrier every wave is done with tile t-1, whose stage receives tile t + NS - 1.
  constexpr int NS = dq_stages<D>();
  constexpr int G = dq_group<D>();
  auto step = [&](auto stage, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    if (NS > 2 && t + 1 < ntiles) wait_vmem_n<(NS - 2) * 2 * LOADS>();
    else wait_vmem();
    barrier();
    if (t + NS - 1 < ntiles) {
      load_tile(rK, t + NS - 1, kst[(S + NS - 1) % NS]);
      load_tile(rV, t + NS - 1, vst[(S + NS - 1) % NS]);
    }
    if (t < n_wave && mine(t)) tile(tix(t), kst[S], vst[S]);
  };
  // Groups of G tiles (G > 1): tiles t .. t+G-1 in stages SB .. SB+G-1 (SB = 0 or G) must have
  // landed; after the barrier every wave is done with the previous group, whose stages receive tiles
  // t+G .. t+2G-1.
  auto group = [&](auto sbase, int t) __attribute__((always_inline)) {
    constexpr int SB = decltype(sbase)::value;
    wait_vmem();
    barrier();
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (t + G + i < ntiles) {
        load_tile(rK, t + G + i, kst[(SB + G + i) % NS]);
        load_tile(rV, t + G + i, vst[(SB + G + i) % NS]);
      }
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (t + i < n_wave && mine(t + i)) tile(tix(t + i), kst[SB + i], vst[SB + i]);
  };
#pragma unroll
  for (int i = 0; i < (G > 1 ? G : NS - 1); ++i)
    if (i < ntiles) {
      load_tile(rK, i, kst[i]);
      load_tile(rV, i, vst[i]);
    }
  // The stationary operands are complete here; saying so (an unconditional use) keeps the compiler
  // from waiting for them -- and, as it cannot tell them apart, for the tile loads in flight --
  // inside the loop.
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    pin(qf[ds]);
    pin(gf[ds]);
  }
  pin(lse2);
  pin(del);
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2 % NS>;
  int t = 0;
  if constexpr (G > 1) {
    using SG = std::integral_constant<int, G % NS>;
    for (; t < ntiles; t += 2 * G) {
      group(S0{}, t);
      if (t + G < ntiles) group(SG{}, t + G);
    }
  } else {
    for (; t + NS - 1 < ntiles; t += NS) {
      step(S0{}, t);
      step(S1{}, t + 1);
      if constexpr (NS > 2) step(S2{}, t + 2);
    }
    if (t < ntiles) step(S0{}, t);
    if (NS > 2 && t + 1 < ntiles) step(S1{}, t + 1);
  }

  // ---- epilogue: dQ = scale acc (bf16, RNE); lane holds query `query`, d = 32 dt + 8 gq + 4 half + 0..3.
  // A store of this layout would write 8-byte pieces of 32 rows per instruction; instead each wave
  // stages its 32 rows in half of a K/V stage (256-byte rows, the tile swizzle) and writes them back as
  // whole 16-byte chunks, 64 / CH full rows per instruction.
  constexpr int RB = kDqRowsPerWave * D * 2;  // bytes of a wave's dQ rows
  static_assert(2 * RB <= TILE && kDqWaves <= 8, "two waves' rows fit in one K or V stage");
  barrier();  // every wave is done with the K/V stages
  {
    const int pair = wave >> 1;
    FA_LDS char* const ep = (pair == 0 ? kst[0] : pair == 1 ? kst[1] : pair == 2 ? vst[0] : vst[1]) + (wave & 1) * RB;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dt + 8 * gq + 4 * half;
        *(FA_LDS bf16x4*)(ep + tile_off<D>(l32, d0)) =
            pack4(acc[dt][4 * gq] * scale, acc[dt][4 * gq + 1] * scale, acc[dt][4 * gq + 2] * scale,
                  acc[dt][4 * gq + 3] * scale);
      }
    constexpr int CHUNKS = kDqRowsPerWave * CH / 64;  // 16-byte chunks per lane
#pragma unroll
    for (int n = 0; n < CHUNKS; ++n) {
      const int pch = n * 64 + lane;
      const int r = pch / CH, c = pch % CH;
      const bf16x8 x = lds_read_b128(ep, tile_off<D>(r, 8 * c));
      if (qw + r < N) *(bf16x8*)(dQ + (row0 + qw + r) * D + 8 * c) = x;
    }
  }
}

template <int D, bool CAUSAL, bool PADDED, bool SPARSE, bool DROP>
hipError_t launch(const Problem& p, const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                  const float* delta, void* dq) {
  const int nqb = (p.N + kDqBr - 1) / kDqBr;
  const int BH = p.B * p.H;
  const Dropout dr{p.drop_k0, p.drop_k1, p.drop_off2, p.drop_t, 256.f / (float)p.drop_t};
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, PADDED, SPARSE, DROP>), dim3((unsigned)(nqb * BH)),
                     dim3(kDqWaves * 64), 0, p.stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                     (const __bf16*)dO, const_cast<float*>(lse2), const_cast<float*>(delta), (__bf16*)dq,
                     (const __bf16*)p.pre_o, p.pre_lse, p.H, p.N, p.scale, p.scale * kLog2e, p.seqlens, p.block_mask,
                     dr, nqb, BH);
  return hipGetLastError();
}

template <int D, bool SPARSE, bool DROP>
hipError_t launch_m(const Problem& p, const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                    const float* delta, void* dq) {
  const bool pad = p.seqlens != nullptr;
  if (p.causal)
    return pad ? launch<D, true, true, SPARSE, DROP>(p, q, k, v, dO, lse2, delta, dq)
               : launch<D, true, false, SPARSE, DROP>(p, q, k, v, dO, lse2, delta, dq);
  return pad ? launch<D, false, true, SPARSE, DROP>(p, q, k, v, dO, lse2, delta, dq)
             : launch<D, false, false, SPARSE, DROP>(p, q, k, v, dO, lse2, delta, dq);
}

template <int D>
hipError_t launch_d(const Problem& p, const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                    const float* delta, void* dq) {
  if (p.dropout) return launch_m<D, false, true>(p, q, k, v, dO, lse2, delta, dq);
  return p.block_mask != nullptr ? launch_m<D, true, false>(p, q, k, v, dO, lse2, delta, dq)
                                 : launch_m<D, false, false>(p, q, k, v, dO, lse2, delta, dq);
}

}  // namespace

int64_t bwd_dq_bf16_grid(int B, int H, int N) { return (int64_t)((N + kDqBr - 1) / kDqBr) * B * H; }

hipError_t launch_bwd_dq_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO, void* dq,
                              const void* workspace) {
  const BwdWorkspace ws = bwd_workspace_layout(p.B, p.H, p.N, p.d, true);
  const float* delta = (const float*)((const char*)workspace + ws.delta_off);
  const float* lse2 = (const float*)((const char*)workspace + ws.lse2_off);
  return p.d == 64 ? launch_d<64>(p, q, k, v, dO, lse2, delta, dq) : launch_d<128>(p, q, k, v, dO, lse2, delta, dq);
}

}  // namespace fa
