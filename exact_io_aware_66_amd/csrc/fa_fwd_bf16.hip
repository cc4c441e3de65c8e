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
//   * a wave owns 32 query rows and fits in 256 registers, so two waves share each SIMD and cover
//     each other's stalls.  Dense d = 128: one workgroup of 8 waves (256 query rows) per compute
//     unit, so each K/V tile reaches the unit's LDS once for 256 rows.  d = 64 and block-sparse
//     masks: workgroups of 4 waves (128 rows, the mask's block), two per compute unit (measured:
//     the 8-wave form is 3 % faster at d = 128 and 3-7 % slower at d = 64); dense d = 64 without
//     dropout: three per compute unit (a wave within 168 registers, K and V^T fragments read one
//     step ahead; measured: -7 % forward time at N = 1024, -1 % at N = 65536);
//   * Q of the wave stays in registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16);
//     each lane holds one query column of the score tile, so the row max/sum are in-lane (the two
//     lane halves hold different keys of the same queries and are combined once, at the end);
//   * K and V tiles of 64 keys stream through two double-buffered LDS rings with direct
//     buffer->LDS 16-byte loads (rows past N read as zeros), one tile ahead;
//   * software pipeline, iteration t (scores of consecutive tiles alternate between two register
//     sets):  S(t+1) = K(t+1) Q^T on the matrix cores while the VALU turns S(t) into P(t) (exp2,
//     bf16 pack, row sums); then O^T += V(t)^T P(t)^T, beside which the VALU finishes P(t) and
//     checks S(t+1) against the running maximum.  Each matrix-core step carries its share of the
//     VALU work, and LDS fragments are read two MFMA steps ahead (V^T through ds_read_b64_tr_b16);
//   * lazy rescaling: the running maximum is only raised when a tile's maximum exceeds it by more
//     than 2^8 (base 2), so p <= 2^8 and the output/normaliser, which share the stale maximum, stay
//     exact; the O rescale therefore runs a few times per row instead of once per tile.  The check
//     for tile t+1 overlaps the P(t) V(t) products, so it is off the critical path.  Normalisation
//     by l is deferred to the epilogue;
//   * tiles with hidden pairs (causal diagonal, key padding, ragged tail) are masked, with an exact
//     maximum update, in a separate form of the iteration;
//   * workgroups are ordered heaviest first (causal) and, when B*H is a multiple of 8, all query
//     blocks of one head go to one XCD (workgroup ids are dealt round-robin over the 8 XCDs), so a
//     head's K/V stays in that XCD's L2.
#include <type_traits>

#include "fa.h"
#include "fa_device.hpp"
#include "fa_launch.hpp"

static_assert(fa::kMaskBlock == FA_MASK_BLOCK && fa::kMaskBlock * fa::kMaxMaskBlocks == FA_MASK_MAX_N,
              "block-mask geometry of the kernels and of the C ABI agree");

namespace fa {
namespace {

constexpr int kFwdRowsPerWave = 32;  // query rows per wave (one 32-column MFMA tile)
constexpr int kFwdBc = 64;           // keys per tile
// Waves per workgroup (the workgroup's query block is 32 rows per wave).
template <int D, bool SPARSE>
constexpr int fwd_waves() { return (D == 128 && !SPARSE) ? 8 : 4; }
constexpr int kFwdMaxBr = 8 * kFwdRowsPerWave;  // largest query block
constexpr int kFwdMinBr = 4 * kFwdRowsPerWave;  // smallest query block (the block-sparse one)
static_assert(kFwdMinBr == fa::kMaskBlock, "a block-sparse query block is one row of mask blocks");
constexpr float kLazyRescale = 8.0f;                 // base-2 headroom before the maximum is raised

// F8: Q, K and V are OCP FP8 E4M3 bytes (the pointers are reinterpreted): S = K Q^T on the FP8
// matrix cores (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulation, exact products), V converted exactly
// to bf16 on its way into LDS, P V as in the bf16 path; the per-tensor descales of Q and K are folded
// into c_log2 and that of V into o_scale.
template <int D, bool CAUSAL, bool PADDED, bool NEG, bool SPARSE, bool DROP, bool F8>
__global__ __launch_bounds__((64 * fwd_waves<D, SPARSE>()), ((D == 64 && !SPARSE && !DROP) ? 3 : 8 / fwd_waves<D, SPARSE>())) void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                          float* __restrict__ LSE, int H, int N, float c_log2,
                                                          const int32_t* __restrict__ seqlens,
                                                          const uint8_t* __restrict__ bmask, Dropout dr, float o_scale,
                                                          int nqb, int BH) {
  static_assert(!F8 || (D == 128 && !SPARSE && !DROP), "the FP8 forward is built for d = 128, dense");
  constexpr int WAVES = fwd_waves<D, SPARSE>();
  constexpr int NT = 64 * WAVES;           // threads per workgroup
  constexpr int BR = WAVES * kFwdRowsPerWave;  // query rows per workgroup
  constexpr int CH = D / 8;                // 16-byte chunks per row
  constexpr int TILE = kFwdBc * D * 2;     // bytes of one K or V tile
  constexpr int LOADS = kFwdBc * CH / NT;  // 16-byte loads per thread per tile
  constexpr int DS = D / 16;                // k-steps of S = K Q^T
  constexpr int DT = D / 32;                // 32-wide d tiles of O^T
  // Separate LDS arrays, each referenced statically, so that the compiler sees which buffer every
  // read addresses.
  __shared__ __attribute__((aligned(1024))) char kbuf0_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0_raw[TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1_raw[TILE];
  FA_LDS char* const kbuf[2] = {(FA_LDS char*)kbuf0_raw, (FA_LDS char*)kbuf1_raw};
  FA_LDS char* const vbuf[2] = {(FA_LDS char*)vbuf0_raw, (FA_LDS char*)vbuf1_raw};
  // block-sparse: the visible key tiles of this query block, in order (two per mask block)
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

  const int L = PADDED ? clamp_len(seqlens, b, N) : N;  // keys >= L are invisible
  const int q0 = qblock * BR;
  const int qw = q0 + wave * kFwdRowsPerWave;
  const int query = qw + l32;
  const int kv_end = CAUSAL ? min(L, q0 + BR) : L;
  int ntiles = (kv_end + kFwdBc - 1) / kFwdBc;  // tiles the workgroup loads
  const int wave_end = CAUSAL ? min(L, qw + kFwdRowsPerWave) : L;
  int n_wave = (wave_end + kFwdBc - 1) / kFwdBc;  // tiles this wave computes (>= 1 when L > 0)
  int n_full = L / kFwdBc;                        // leading tiles with no hidden pair
  if (CAUSAL) n_full = min(n_full, qw / kFwdBc);
  int n_clean = min(n_full, n_wave);
  // Block-sparse: the loop below walks the list of visible tiles instead of tiles 0 .. ntiles-1; the
  // counts become positions in that list (the list is in tile order, so the fully visible tiles are
  // still its head).  A tile is always wholly inside one mask block.
  const FA_LDS uint16_t* const tlist = (const FA_LDS uint16_t*)tlist_raw;
  if constexpr (SPARSE) {
    const int nb = (N + kMaskBlock - 1) / kMaskBlock;
    const uint8_t* brow = bmask + ((int64_t)bh * nb + qblock) * nb;
    if (wave == 0)
      compact_tiles<kMaskBlock / kFwdBc>((FA_LDS uint16_t*)tlist_raw, (FA_LDS int*)&tcount_raw, 0,
                                         (ntiles + 1) / 2, ntiles, [&](int kb) { return brow[kb] != 0 ? 1 : 0; });
    __syncthreads();
    const int n = *(volatile FA_LDS int*)&tcount_raw;
    n_wave = count_below(tlist, n, n_wave);
    n_clean = count_below(tlist, n, n_clean);
    ntiles = n;
  }
  // position t of the walk -> key tile
  auto tix = [&](int t) { return SPARSE ? list_tile(tlist[t]) : t; };

  // Q^T fragments (B operand of S^T = K Q^T): lane holds query `query`, d = 16 ds + 8 half .. +7
  bf16x8 qf[F8 ? 1 : DS];
  // F8: lane holds query `query`, bytes d = 64 m + 32 half .. +31 for k-step m (the same per-lane d
  // set as the K fragment, so the product sums over every d whatever the instruction's k order)
  constexpr int DM = D / 64;
  i32x8 qf8[F8 ? DM : 1];
  if constexpr (F8) {
    const uint8_t* q8 = (const uint8_t*)Q + row0 * D;
#pragma unroll
    for (int m = 0; m < DM; ++m) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (query < N) {
        a = *(const u32x4*)(q8 + (int64_t)query * D + 64 * m + 32 * half);
        b = *(const u32x4*)(q8 + (int64_t)query * D + 64 * m + 32 * half + 16);
      }
      qf8[m] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
  } else {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      if (query < N) {
        qf[ds] = *(const bf16x8*)(Qh + (int64_t)query * D + 16 * ds + 8 * half);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ds][e] = (__bf16)0.f;
      }
    }
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
  // Base-2 running maximum (identical in both lane halves), the maximum P is taken against (0 while
  // the row has seen no visible key), and the per-lane partial normaliser (this lane's keys).
  float m_run = -INFINITY, m_p = 0.f, l_run = 0.f;

  // K/V tile loads: buffer loads straight into LDS; rows past N read as zeros (the buffer ends at
  // the head's last row; those keys are masked).  K and V tiles share the per-lane byte offsets,
  // which are loop-invariant.
  uint32_t voff[LOADS];
#pragma unroll
  for (int n = 0; n < LOADS; ++n) {
    const int p = (n * WAVES + wave) * 64 + lane;
    const int r = p / CH;
    const int c = (p % CH) ^ swz<D>(r);
    voff[n] = (uint32_t)(r * D + 8 * c) * 2;
  }
  // One buffer resource per tensor over the whole head (built once): a tile's byte offset goes into the
  // per-lane offset, which the range check covers, so rows past N still read as zeros.
  const u32x4 rK = make_rsrc(Kh, N * D * 2), rV = make_rsrc(Vh, N * D * 2);
  auto load_tile = [&](const u32x4& rs, int t, FA_LDS char* dst) {
    const uint32_t tb = (uint32_t)tix(t) * kFwdBc * D * 2;
#pragma unroll
    for (int n = 0; n < LOADS; ++n) bload_lds16(rs, voff[n] + tb, dst + (n * WAVES + wave) * 1024);
  };
  // F8: K tiles of 64 rows x D bytes (128-byte rows, swizzled like 64-column bf16 rows), loaded
  // straight into LDS; V tiles loaded into registers, converted to bf16 and stored in the bf16 tile
  // layout the P V products read.
  constexpr int LOADS8 = kFwdBc * (D / 16) / NT;
  uint32_t voff8[F8 ? LOADS8 : 1];
  if constexpr (F8) {
#pragma unroll
    for (int n = 0; n < LOADS8; ++n) {
      const int p = (n * WAVES + wave) * 64 + lane;
      const int r = p / (D / 16);
      const int c = (p % (D / 16)) ^ swz<64>(r);
      voff8[n] = (uint32_t)(r * D + 16 * c);
    }
  }
  auto load_k8 = [&](int t, FA_LDS char* dst) {
    const uint8_t* k8 = (const uint8_t*)K + (row0 + (int64_t)t * kFwdBc) * D;
    const u32x4 rs = make_rsrc(k8, (N - t * kFwdBc) * D);
#pragma unroll
    for (int n = 0; n < LOADS8; ++n) bload_lds16(rs, voff8[n], dst + (n * WAVES + wave) * 1024);
  };
  auto k8_off = [&](int row, int c) { return (uint32_t)(row * D + 16 * (c ^ swz<64>(row))); };
  u32x4 vreg[2];  // F8: this thread's 16-byte chunks of the next V tile (512 / NT of them)
  auto load_v8 = [&](int t) {
    const uint8_t* v8 = (const uint8_t*)V + row0 * D;
#pragma unroll
    for (int n = 0; n < 512 / NT; ++n) {
      const int p = n * NT + (int)threadIdx.x;
      const int r = min(t * kFwdBc + (p >> 3), N - 1);  // rows past N: any finite values (masked keys)
      vreg[n] = *(const u32x4*)(v8 + (int64_t)r * D + 16 * (p & 7));
    }
  };
  auto store_v8 = [&](FA_LDS char* dst) {
#pragma unroll
    for (int n = 0; n < 512 / NT; ++n) {
      const int p = n * NT + (int)threadIdx.x;
      const int r = p >> 3, c8 = p & 7;
      bf16x8 half8[2];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)vreg[n][w], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)vreg[n][w], true);
        half8[w >> 1][4 * (w & 1) + 0] = (__bf16)lo[0];
        half8[w >> 1][4 * (w & 1) + 1] = (__bf16)lo[1];
        half8[w >> 1][4 * (w & 1) + 2] = (__bf16)hi[0];
        half8[w >> 1][4 * (w & 1) + 3] = (__bf16)hi[1];
      }
      *(FA_LDS bf16x8*)(dst + tile_off<D>(r, 16 * c8)) = half8[0];
      *(FA_LDS bf16x8*)(dst + tile_off<D>(r, 16 * c8 + 8)) = half8[1];
    }
  };

  // S^T of two consecutive tiles: s[set][kt], lane = query column, rows = keys 32 kt + 8 (r/4) +
  // 4 half + r%4 of the tile
  f32x16 s[2][2];
  bf16x8 pn[4];  // P(t) packed to bf16 (B operand of O^T += V^T P^T), one per 16-key k-step
  bf16x2 pk[4][4];
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  const int g = lane >> 4, j = lane & 15;
  const int vrow = 4 * (g >> 1) + (j >> 2);

  // Work units of the VALU, placed between the MFMAs of the matrix-core phases:
  //   punit(set, ks, e): two elements of P(t) (k-step ks, pair e) = exp2(s cf - m_p), their bf16
  //     pack and row sum (v_dot2_f32_bf16 on the packed values, so l sums exactly the weights used);
  //   xunit(set, u): four scores of the next tile into the running extreme ext (max, or min for a
  //     negative scale) for the lazy check.
  // Dropout: keep words of the lane's query for the current tile's 32-key half kt (computed as a work
  // unit before the P units that need them); l sums every probability, P V only the kept ones (the
  // 256/t scale of the kept ones is applied to O in the epilogue).
  u32x4 kwd = {};
  auto dunit = [&](int t, int kt) {
    if constexpr (DROP) kwd = dropout_words<true>(dr, (uint32_t)bh, query, 2 * tix(t) + kt, half);
  };
  auto punit = [&](int set, int ks, int e, float cf) {
    const int kt = ks >> 1, r = 8 * (ks & 1) + 2 * e;
    const f32x2 two = {fast_exp2(fmaf(s[set][kt][r], cf, -m_p)), fast_exp2(fmaf(s[set][kt][r + 1], cf, -m_p))};
    pk[ks][e] = __builtin_convertvector(two, bf16x2);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(pk[ks][e], ones, l_run, false);
    if constexpr (DROP) {
      const uint32_t w = kwd[r >> 2];
      const f32x2 kept = {dropout_keep(dr, w, r & 3) ? two[0] : 0.f, dropout_keep(dr, w, (r & 3) + 1) ? two[1] : 0.f};
      pk[ks][e] = __builtin_convertvector(kept, bf16x2);
    }
    if (e == 3)
      pn[ks] = cat(__builtin_shufflevector(pk[ks][0], pk[ks][1], 0, 1, 2, 3),
                   __builtin_shufflevector(pk[ks][2], pk[ks][3], 0, 1, 2, 3));
  };
  float ext = 0.f;
  auto xunit = [&](int set, int u) {
    const int kt = u >> 2, r = 4 * (u & 3);
    const f32x16& v = s[set][kt];
    if (u == 0) ext = v[0];
    ext = NEG ? fminf(fminf(ext, v[r]), fminf(v[r + 1], fminf(v[r + 2], v[r + 3])))
              : fmaxf(fmaxf(ext, v[r]), fmaxf(v[r + 1], fmaxf(v[r + 2], v[r + 3])));
  };

  // S^T(tile in kb) = K Q^T into s[set]: DS k-steps of 2 MFMAs, K fragments read KRA k-steps ahead;
  // `between(ds)` places VALU work after the MFMAs of k-step ds
  auto scores = [&](int set, const FA_LDS char* kb, auto&& between) __attribute__((always_inline)) {
    if constexpr (F8) {
      // 2 DM FP8 MFMAs (K = 64 each); the DS VALU slots are spread two per MFMA
      i32x8 a8[DM][2];
#pragma unroll
      for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int row = 32 * kt + l32;
          const bf16x8 x = lds_read_b128(kb, k8_off(row, 4 * m + 2 * half));
          const bf16x8 y = lds_read_b128(kb, k8_off(row, 4 * m + 2 * half + 1));
          const u32x4 xu = __builtin_bit_cast(u32x4, x), yu = __builtin_bit_cast(u32x4, y);
          a8[m][kt] = i32x8{(int)xu[0], (int)xu[1], (int)xu[2], (int)xu[3], (int)yu[0], (int)yu[1], (int)yu[2], (int)yu[3]};
        }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[set][kt] = zero16();
#pragma unroll
      for (int m = 0; m < DM; ++m)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          __builtin_amdgcn_sched_barrier(0);
          s[set][kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[m][kt], qf8[m], s[set][kt], 0, 0, 0, 0, 0, 0);
          const int slot = 2 * (2 * m + kt) * DS / (4 * DM);
#pragma unroll
          for (int z = 0; z < DS / (2 * DM); ++z) between(slot + z);
        }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    constexpr int KRA = 1;  // K fragments read KRA k-steps ahead
    bf16x8 kf[KRA + 1][2];
    auto rd = [&](int ds, bf16x8 (&f)[2]) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) f[kt] = lds_read_b128(kb, tile_off<D>(32 * kt + l32, 16 * ds + 8 * half));
    };
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[set][kt] = zero16();
#pragma unroll
    for (int ds = 0; ds < KRA; ++ds) rd(ds, kf[ds]);
    // Raised issue priority while this wave feeds S to the matrix cores, so that of two waves on a SIMD in
    // different phases the one with score products goes first (measured: -3 % forward at d = 64,
    // N = 65536, where the two workgroups of a compute unit drift apart; no change elsewhere).
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      __builtin_amdgcn_sched_barrier(0);
      if (ds + KRA < DS) rd(ds + KRA, kf[(ds + KRA) % (KRA + 1)]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[set][kt] = mfma32x32x16(kf[ds % (KRA + 1)][kt], qf[ds], s[set][kt]);
      between(ds);
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // O^T += V^T P^T over the tile in vb, k-step outermost: 4 DT MFMAs.  V^T fragment of product i
  // (dt = i % DT, ks = i / DT): lane (d = 32 dt + l32, half) needs keys 16 ks + 4 half + 0..3 and
  // 16 ks + 8 + 4 half + 0..3, the key order of pn; two transposing reads supply them (bases for
  // rows vrow and vrow + 8, compile-time offsets of 16 rows).  The fragments run VRA products ahead
  // in a ring of VRA + 1; the first VRA are read by the caller during the score products before it
  // (pv_head), so the matrix cores do not wait for them at the phase change.  `between(i)` follows
  // MFMA i.
  constexpr int NPV = 4 * DT;
  constexpr int VRA = (D == 64) ? 1 : 3;  // V^T fragments read VRA products ahead
  bf16x8 vf[VRA + 1];
  auto pv_rd = [&](const FA_LDS char* vb, int i) __attribute__((always_inline)) {
    const int ks = i / DT, dt = i % DT;
    const uint32_t off0 = tile_off<D>(vrow, 32 * dt + 16 * (g & 1) + 4 * (j & 3)) + ks * 16 * D * 2;
    const uint32_t off8 = tile_off<D>(vrow + 8, 32 * dt + 16 * (g & 1) + 4 * (j & 3)) + ks * 16 * D * 2;
    vf[i % (VRA + 1)] = cat(lds_read_tr(vb, off0), lds_read_tr(vb, off8));
  };
  auto pv_head = [&](const FA_LDS char* vb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < VRA; ++i) pv_rd(vb, i);
  };
  auto pv = [&](const FA_LDS char* vb, auto&& between) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + VRA < NPV) pv_rd(vb, i + VRA);
      acc[i % DT] = mfma32x32x16(vf[i % (VRA + 1)], pn[i / DT], acc[i % DT]);
      between(i);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // Exact update for a tile with hidden pairs (scores in s[set]): hidden scores to -inf, the rest
  // scaled to the base-2 domain in place; raise the maximum to the tile's.  Returns the factor O and
  // l must be multiplied by (1 when the maximum is unchanged).
  auto mask_update = [&](int set, int t) -> float {
    // element (kt, r) holds key key0 + 32 kt + 8 (r / 4) + 4 half + r % 4: visible iff its offset
    // 32 kt + 8 (r / 4) + r % 4, a constant per register, is below one per-lane limit
    const int lim = (CAUSAL ? min(L, query + 1) : L) - (tix(t) * kFwdBc + 4 * half);
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool vis = (32 * kt + 8 * (r >> 2) + (r & 3)) < lim;
        const float v = vis ? s[set][kt][r] * c_log2 : -INFINITY;
        s[set][kt][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_p - m_use);
    m_run = m_new;
    m_p = m_use;
    return alpha;
  };
  // Exact maximum of a fully visible tile (the first one of the wave): no rescale needed before it.
  auto exact_update = [&](int set) -> float {
    float mx = s[set][0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = NEG ? fminf(mx, s[set][kt][r]) : fmaxf(mx, s[set][kt][r]);
    mx = (NEG ? min_halves(mx) : max_halves(mx)) * c_log2;
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_p - m_new);
    m_run = m_new;
    m_p = m_new;
    return alpha;
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    l_run *= alpha;
  };

  // ---- prologue: K(0), K(1), V(0); S(0) and its exact update
  if (ntiles > 0) {
    if constexpr (F8) {
      load_k8(0, kbuf[0]);
      if (ntiles > 1) load_k8(1, kbuf[1]);
      load_v8(0);
      store_v8(vbuf[0]);
    } else {
      load_tile(rK, 0, kbuf[0]);
      if (ntiles > 1) load_tile(rK, 1, kbuf[1]);
      load_tile(rV, 0, vbuf[0]);
    }
  }
  wait_vmem();
  if constexpr (F8) barrier_lds();
  else barrier();
  // The Q fragments are complete here; saying so (an unconditional use) keeps the compiler from
  // waiting for them -- and, as it cannot tell them apart, for the tile loads in flight -- inside
  // the loop.
  if constexpr (F8) {
#pragma unroll
    for (int m = 0; m < DM; ++m) pin(qf8[m]);
  } else {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) pin(qf[ds]);
  }
  if (n_wave > 0) {
    scores(0, kbuf[0], [](int) {});
    if (n_clean > 0) exact_update(0);
    else mask_update(0, 0);
  }

  // Iteration t (every wave runs t = 0 .. ntiles-1, one barrier each; V(t) and K(t+1) were loaded
  // one iteration ahead).  S(t) is in s[t % 2] (scaled and masked in place when tile t has hidden
  // pairs, else raw: cf tells which), and the maximum for P(t) is settled.
  //   phase 1:  S(t+1) = K(t+1) Q^T into the other set  ||  P(t), k-steps 0..2; first V(t)^T fragments
  //   phase 2:  O += V(t)^T P(t), k-steps 0 .. 3          ||  P(t), k-step 3, then the extreme of S(t+1)
  //   then the lazy check for tile t+1 (raise the maximum, rescale O and l), or, when tile t+1 has
  //   hidden pairs, its mask and exact update.
  // The forms differ in the next tile (fully visible, with hidden pairs, none) and in whether the
  // set and buffer indices are compile-time (the unrolled loop over fully visible tiles) or picked
  // at run time (a few tiles per wave).  kIdle iterations only load for the workgroup.
  constexpr int kNextClean = 0, kNextMasked = 1, kNextNone = 2, kIdle = 3;
  auto step = [&](auto next_tag, int t, int cur, const float cf) __attribute__((always_inline)) {
    constexpr int NEXT = decltype(next_tag)::value;
    const int nxt = cur ^ 1;
    wait_vmem();  // K(t+1) and V(t), issued one iteration ago, have landed
    if constexpr (F8) barrier_lds();  // (and the bf16 V(t) written to LDS at the end of the last one)
    else barrier();
    if constexpr (F8) {
      if (t + 2 < ntiles) load_k8(t + 2, kbuf[cur]);
      if (t + 1 < ntiles) load_v8(t + 1);  // converted into vbuf[nxt] at the end of this iteration
    } else {
      if (t + 2 < ntiles) load_tile(rK, t + 2, kbuf[cur]);  // over K(t), read in iteration t-1
      if (t + 1 < ntiles) load_tile(rV, t + 1, vbuf[nxt]);  // over V(t-1), read in iteration t-1
    }
    if constexpr (NEXT == kIdle) {
      if constexpr (F8) {
        if (t + 1 < ntiles) store_v8(vbuf[nxt]);
      }
      return;
    } else {
      // phase 1: 12 P units over the DS k-steps of S(t+1) (P only when there is no next tile); the
      // first V^T fragments of phase 2 are read two k-steps before its end
      auto ph1 = [&](int ds) {
#pragma unroll
        for (int x = 0; x < 12; ++x)
          if (x * DS / 12 == ds) {
            if (x == 0) dunit(t, 0);
            if (x == 8) dunit(t, 1);
            punit(cur, x / 4, x % 4, cf);
          }
        if (ds == DS - 2) pv_head(vbuf[cur]);
      };
      if constexpr (NEXT != kNextNone) {
        scores(nxt, kbuf[nxt], ph1);
      } else {
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) ph1(ds);
      }
      // phase 2: 4 DT MFMAs; in the first half 4 P units then 4 extreme units, in the second half 4
      // extreme units
      pv(vbuf[cur], [&](int i) {
        if (i < 2 * DT) {
#pragma unroll
          for (int x = 0; x < 8; ++x)
            if (x * 2 * DT / 8 == i) {
              if (x < 4) punit(cur, 3, x, cf);
              else if (NEXT == kNextClean) xunit(nxt, x - 4);
            }
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x)
            if (x * 2 * DT / 4 == i - 2 * DT && NEXT == kNextClean) xunit(nxt, 4 + x);
        }
      });
      if constexpr (NEXT == kNextClean) {
        // Lazy check.  c_log2 scales monotonically, so some lane's partial extreme (its half's keys)
        // passes the threshold exactly when the extreme over both halves does: the test needs no
        // exchange between the halves, only the (rare) raise does.
        if (__builtin_amdgcn_ballot_w64(ext * c_log2 > m_run + kLazyRescale) != 0) {
          const float tm = (NEG ? min_halves(ext) : max_halves(ext)) * c_log2;
          const float m_new = fmaxf(m_run, tm);
          const float alpha = fast_exp2(m_p - m_new);
          m_run = m_new;
          m_p = m_new;
          rescale(alpha);
        }
      } else if constexpr (NEXT == kNextMasked) {
        const float alpha = mask_update(nxt, t + 1);
        if (__builtin_amdgcn_readfirstlane(__any(alpha != 1.f))) rescale(alpha);
      }
      if constexpr (F8) {  // V(t+1) into the other buffer (read from the next iteration on)
        if (t + 1 < ntiles) store_v8(vbuf[nxt]);
      }
    }
  };

  using NC = std::integral_constant<int, kNextClean>;
  // fully visible tile followed by a fully visible tile: compile-time sets and buffers
  int t = 0;
  const int n_cc = n_clean - 1;  // iterations t with tiles t and t+1 both fully visible
  for (; t + 1 < n_cc; t += 2) {
    step(NC{}, t, 0, c_log2);
    step(NC{}, t + 1, 1, c_log2);
  }
  if (t < n_cc) {
    step(NC{}, t, 0, c_log2);
    ++t;
  }
  // the rest: S(t) is moved to set 0 first, and every remaining form keeps it there (S(t+1) is
  // computed into set 1 and moved to set 0 at the end)
  if (t & 1) {
    s[0][0] = s[1][0];
    s[0][1] = s[1][1];
  }
  auto run = [&](auto next_tag, int t) __attribute__((always_inline)) {
    const bool odd = t & 1;
    FA_LDS char* kb_cur = odd ? kbuf[1] : kbuf[0];
    FA_LDS char* kb_nxt = odd ? kbuf[0] : kbuf[1];
    FA_LDS char* vb_cur = odd ? vbuf[1] : vbuf[0];
    FA_LDS char* vb_nxt = odd ? vbuf[0] : vbuf[1];
    constexpr int NEXT = decltype(next_tag)::value;
    const float cf = t < n_clean ? c_log2 : 1.f;
    wait_vmem();
    if constexpr (F8) barrier_lds();
    else barrier();
    if constexpr (F8) {
      if (t + 2 < ntiles) load_k8(t + 2, kb_cur);
      if (t + 1 < ntiles) load_v8(t + 1);
    } else {
      if (t + 2 < ntiles) load_tile(rK, t + 2, kb_cur);
      if (t + 1 < ntiles) load_tile(rV, t + 1, vb_nxt);
    }
    if constexpr (NEXT != kIdle) {
      auto ph1 = [&](int ds) {
#pragma unroll
        for (int x = 0; x < 12; ++x)
          if (x * DS / 12 == ds) {
            if (x == 0) dunit(t, 0);
            if (x == 8) dunit(t, 1);
            punit(0, x / 4, x % 4, cf);
          }
        if (ds == DS - 2) pv_head(vb_cur);
      };
      if constexpr (NEXT == kNextMasked) {
        scores(1, kb_nxt, ph1);
      } else {
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) ph1(ds);
      }
      pv(vb_cur, [&](int i) {
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (x * 2 * DT / 4 == i) punit(0, 3, x, cf);
      });
      if constexpr (NEXT == kNextMasked) {
        const float alpha = mask_update(1, t + 1);
        if (__builtin_amdgcn_readfirstlane(__any(alpha != 1.f))) rescale(alpha);
        s[0][0] = s[1][0];
        s[0][1] = s[1][1];
      }
    }
    if constexpr (F8) {
      if (t + 1 < ntiles) store_v8(vb_nxt);
    }
  };
  for (; t + 1 < n_wave; ++t) run(std::integral_constant<int, kNextMasked>{}, t);
  if (t < n_wave) run(std::integral_constant<int, kNextNone>{}, t++);
  for (; t < ntiles; ++t) run(std::integral_constant<int, kIdle>{}, t);

  // ---- epilogue: O = acc / l (bf16, RNE); LSE = (m + log2 l) ln 2.  A store of the accumulator layout
  // would write 8-byte pieces of 32 rows per instruction; instead each wave stages its 32 rows of O in
  // half of a K or V buffer (256-byte rows, the tile swizzle) and writes them back as whole 16-byte
  // chunks, 64 / CH full rows per instruction.
  constexpr int RB = kFwdRowsPerWave * D * 2;  // bytes of a wave's O rows
  static_assert(2 * RB <= TILE && WAVES <= 8, "two waves' rows fit in one K or V buffer");
  barrier();  // every wave is done with the K/V buffers
  {
    const float l = add_halves(l_run);
    const bool has = l > 0.f;
    const float inv = has ? (DROP ? dr.scale : 1.f) * (F8 ? o_scale : 1.f) / l : 0.f;
    if (query < N && half == 0) LSE[row0 + query] = has ? (m_p + __log2f(l)) * kLn2 : -INFINITY;
    const int pair = wave >> 1;
    FA_LDS char* const ep = (pair == 0 ? kbuf[0] : pair == 1 ? kbuf[1] : pair == 2 ? vbuf[0] : vbuf[1]) + (wave & 1) * RB;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dt + 8 * gq + 4 * half;
        *(FA_LDS bf16x4*)(ep + tile_off<D>(l32, d0)) =
            pack4(acc[dt][4 * gq] * inv, acc[dt][4 * gq + 1] * inv, acc[dt][4 * gq + 2] * inv, acc[dt][4 * gq + 3] * inv);
      }
    constexpr int CHUNKS = kFwdRowsPerWave * CH / 64;  // 16-byte chunks per lane
#pragma unroll
    for (int n = 0; n < CHUNKS; ++n) {
      const int pch = n * 64 + lane;
      const int r = pch / CH, c = pch % CH;
      const bf16x8 x = lds_read_b128(ep, tile_off<D>(r, 8 * c));
      if (qw + r < N) *(bf16x8*)(O + (row0 + qw + r) * D + 8 * c) = x;
    }
  }
}

template <int D, bool CAUSAL, bool PADDED, bool NEG, bool SPARSE, bool DROP, bool F8 = false>
hipError_t launch(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  constexpr int WAVES = fwd_waves<D, SPARSE>();
  constexpr int BR = WAVES * kFwdRowsPerWave;
  const int nqb = (p.N + BR - 1) / BR;
  const int BH = p.B * p.H;
  const float c_log2 = p.scale * kLog2e * (F8 ? p.fp8_qk_descale : 1.f);
  const Dropout dr{p.drop_k0, p.drop_k1, p.drop_off2, p.drop_t, 256.f / (float)p.drop_t};
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, PADDED, NEG, SPARSE, DROP, F8>), dim3((unsigned)(nqb * BH)), dim3(64 * WAVES), 0, p.stream,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, p.H, p.N, c_log2,
                     p.seqlens, p.block_mask, dr, F8 ? p.fp8_v_descale : 1.f, nqb, BH);
  return hipGetLastError();
}

template <int D, bool NEG, bool SPARSE, bool DROP>
hipError_t launch_mask(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  const bool pad = p.seqlens != nullptr;
  if (p.causal)
    return pad ? launch<D, true, true, NEG, SPARSE, DROP>(p, q, k, v, o, lse)
               : launch<D, true, false, NEG, SPARSE, DROP>(p, q, k, v, o, lse);
  return pad ? launch<D, false, true, NEG, SPARSE, DROP>(p, q, k, v, o, lse)
             : launch<D, false, false, NEG, SPARSE, DROP>(p, q, k, v, o, lse);
}

template <int D>
hipError_t launch_d(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  if (p.dropout)  // (dense attention only: the C ABI has no entry point that combines the two)
    return p.scale < 0.f ? launch_mask<D, true, false, true>(p, q, k, v, o, lse)
                         : launch_mask<D, false, false, true>(p, q, k, v, o, lse);
  if (p.block_mask != nullptr)
    return p.scale < 0.f ? launch_mask<D, true, true, false>(p, q, k, v, o, lse)
                         : launch_mask<D, false, true, false>(p, q, k, v, o, lse);
  return p.scale < 0.f ? launch_mask<D, true, false, false>(p, q, k, v, o, lse)
                       : launch_mask<D, false, false, false>(p, q, k, v, o, lse);
}

}  // namespace

// The largest grid any forward instantiation launches (the 128-row query blocks).
int64_t fwd_bf16_grid(int B, int H, int N) { return (int64_t)((N + kFwdMinBr - 1) / kFwdMinBr) * B * H; }

hipError_t launch_fwd_fp8(const Problem& p, const void* q8, const void* k8, const void* v8, void* o, float* lse) {
  const bool pad = p.seqlens != nullptr, neg = p.scale < 0.f;
  if (p.causal) {
    if (pad) return neg ? launch<128, true, true, true, false, false, true>(p, q8, k8, v8, o, lse)
                        : launch<128, true, true, false, false, false, true>(p, q8, k8, v8, o, lse);
    return neg ? launch<128, true, false, true, false, false, true>(p, q8, k8, v8, o, lse)
               : launch<128, true, false, false, false, false, true>(p, q8, k8, v8, o, lse);
  }
  if (pad) return neg ? launch<128, false, true, true, false, false, true>(p, q8, k8, v8, o, lse)
                      : launch<128, false, true, false, false, false, true>(p, q8, k8, v8, o, lse);
  return neg ? launch<128, false, false, true, false, false, true>(p, q8, k8, v8, o, lse)
             : launch<128, false, false, false, false, false, true>(p, q8, k8, v8, o, lse);
}

hipError_t launch_fwd_bf16(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  return p.d == 64 ? launch_d<64>(p, q, k, v, o, lse) : launch_d<128>(p, q, k, v, o, lse);
}

}  // namespace fa
