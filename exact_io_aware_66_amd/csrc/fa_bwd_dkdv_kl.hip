// dK and dV of the backward at d = 128 for attention without a block mask (dense, and with fused
// dropout), with two waves per SIMD: the arithmetic of bwd_dkdv_kernel (fa_bwd_bf16.hip) in the same
// order, so the results are bitwise the same, with K held in LDS instead of registers.
//
// A wave of bwd_dkdv_kernel keeps K and V of its 32 keys, dK^T and dV^T and two sets of S and dP in
// about 400 registers, one wave per SIMD.  Here K of the workgroup's 256 keys sits in LDS (64 KiB,
// read as the B operand of S = Q K^T at each k-step), V stays in registers, and one set of S and dP
// is computed, turned into P and dS and consumed per query tile, so a wave needs at most 256
// registers and 8 waves (two per SIMD) share a compute unit.  Per tile: S = Q K^T and
// dP - D = dO V^T - D (v_mfma_f32_32x32x16_bf16, dP starting from -D), P = exp2(S scale log2 e -
// LSE log2 e), dS = P (dP - D), packed to bf16, then dV^T += dO^T P and dK^T += Q^T dS (dO^T and Q^T
// through transposing LDS reads), query halves in order, P and dS of the second half computed beside
// the first half's products; the other wave of the SIMD fills the gaps between a wave's phases.
// Query tiles of 32 rows stream through a four-stage LDS ring fetched three tiles ahead, one barrier
// per tile.  With dropout, the keep decisions of each 32 x 32 block are regenerated as in
// bwd_dkdv_kernel (one Philox call per lane in the generator's query-major layout, a byte transpose
// through the wave's LDS block); the dropout instantiations keep part of their state in scratch
// memory, the others none.  NOTE-005: FlashAttention, "Method" (the recomputation of the attention
// block in the backward); dropout: promptingindex page, "Why attention is memory-bound, not
// compute-bound" (dropout among the steps of the attention chain).
#include <type_traits>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kWkl = 8;               // waves per workgroup (two per SIMD)
constexpr int kKeysKl = 32;           // keys per wave
constexpr int kBcKl = kWkl * kKeysKl;  // 256 keys per workgroup
constexpr int kBrKl = 32;             // query rows per tile

template <bool CAUSAL, bool PADDED, bool DROP>
__global__ __launch_bounds__(kWkl * 64, 1) void bwd_dkdv_kl_kernel(const __bf16* __restrict__ Q,
                                                                   const __bf16* __restrict__ K,
                                                                   const __bf16* __restrict__ V,
                                                                   const __bf16* __restrict__ dO,
                                                                   const float* __restrict__ LSE2,
                                                                   const float* __restrict__ NDELTA,
                                                                   __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                                                                   int H, int N, float scale, float c_log2,
                                                                   const int32_t* __restrict__ seqlens, Dropout dr,
                                                                   int BH) {
  constexpr int D = 128;
  constexpr int DS = D / 16;                     // k-steps over d
  constexpr int DT = D / 32;                     // 32-wide d tiles
  constexpr int QTILE = kBrKl * D * 2;           // bytes of a Q or dO tile
  constexpr int STAGE = 2 * QTILE + kWkl * 256;  // Q | dO | a 256-byte statistics slot per wave
  constexpr int VPT = 3;                         // vector-memory instructions per wave and tile
  __shared__ __attribute__((aligned(1024))) char kst_raw[kBcKl * D * 2];
  __shared__ __attribute__((aligned(1024))) char st0_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char st1_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char st2_raw[STAGE];
  __shared__ __attribute__((aligned(1024))) char st3_raw[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t drop_raw[DROP ? kWkl * 1024 : 16];
  const FA_LDS char* const kst = (const FA_LDS char*)kst_raw;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int g16 = lane >> 4, j16 = lane & 15;

  // ---- work item: (block of 256 keys, batch*head), ascending key blocks first (heaviest under the
  // causal mask); all key blocks of a head on one XCD when B*H is a multiple of 8
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
  const int L = PADDED ? clamp_len(seqlens, b, N) : N;
  const int k0 = kblock * kBcKl;
  const int kw = k0 + wave * kKeysKl;
  const int my_key = kw + l32;

  f32x16 dvt[DT], dkt[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dvt[dt] = zero16();
    dkt[dt] = zero16();
  }

  if (k0 < L) {
    // ---- V of this wave's keys in registers (B operand of dP = dO V^T): lane key my_key, d = 16 ds +
    // 8 half .. +7; K of the workgroup's keys into LDS (row = key - k0, the tile swizzle; rows past N
    // read as zeros)
    bf16x8 vb[DS];
    {
      const int key = min(my_key, N - 1);  // keys past N are never written back
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) vb[ds] = *(const bf16x8*)(V + (row0 + key) * D + 16 * ds + 8 * half);
    }
    const u32x4 rk = make_rsrc(K + row0 * D, N * D * 2);
#pragma unroll
    for (int n = 0; n < kBcKl * 16 / (kWkl * 64); ++n) {
      const int p = (n * kWkl + wave) * 64 + lane;
      const int r = p >> 4;
      const int ch = (p & 15) ^ swz<D>(r);
      bload_lds16(rk, (uint32_t)((k0 + r) * D + 8 * ch) * 2, (FA_LDS char*)kst_raw + (n * kWkl + wave) * 1024);
    }

    const int nqt = (N + kBrKl - 1) / kBrKl;
    const int it0 = CAUSAL ? k0 / kBrKl : 0;
    const int count = nqt - it0;  // query tiles this key block visits (>= 1)
    // This wave's keys see query tiles from tskip on; the four from tskip on take the masked form (the
    // tiles the 128-key workgroups of bwd_dkdv_kernel treat so), the rest the clean one.
    const int tskip = CAUSAL ? 4 * (wave >> 2) : 0;

    // Query tiles: one 16-byte load per thread for Q and for dO (rows past N read as zeros); wave w
    // fetches 64 rows of LSE log2 e (w even) or -D (w odd) into its statistics slot.
    const int p = wave * 64 + lane;
    const int pr = p >> 4;
    const uint32_t voff = (uint32_t)(pr * D + 8 * ((p & 15) ^ swz<D>(pr))) * 2;
    const u32x4 rq = make_rsrc(Q + row0 * D, N * D * 2);
    const u32x4 rg = make_rsrc(dO + row0 * D, N * D * 2);
    const u32x4 rs = make_rsrc(((wave & 1) ? NDELTA : LSE2) + row0, N * 4);
    auto load_tile = [&](int u, FA_LDS char* dst) {
      const int qbase = (it0 + u) * kBrKl;
      const uint32_t tb = (uint32_t)qbase * D * 2;
      bload_lds16(rq, voff + tb, dst + wave * 1024);
      bload_lds16(rg, voff + tb, dst + QTILE + wave * 1024);
      bload_lds4(rs, (uint32_t)(qbase + lane) * 4, dst + 2 * QTILE + wave * 256);
    };
    const int trow = 4 * (g16 >> 1) + (j16 >> 2);

    // One tile u from stage st.  MASK: the masked form (std::true_type, std::false_type, or a run-time
    // bool for the tiles near the causal diagonal, where the form differs between waves).
    auto step = [&](auto mask, const FA_LDS char* st, int u) __attribute__((always_inline)) {
      // Dropout keep words of tile u in this kernel's layout (lane = key, the 16 queries of its half): each
      // lane draws the words of one query (the generator's layout), writes the bytes key-major into the
      // wave's LDS block and reads back the 4 words of its own key
      u32x4 kwt = {};
      if constexpr (DROP) {
        FA_LDS uint8_t* mt = (FA_LDS uint8_t*)drop_raw + wave * 1024;
        const u32x4 w = dropout_words(dr, (uint32_t)bh, (it0 + u) * kBrKl + l32, kw / 32, half);
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) mt[(8 * g + 4 * half + e) * 32 + l32] = (uint8_t)(w[g] >> (8 * e));
#pragma unroll
        for (int g = 0; g < 4; ++g) kwt[g] = *(const FA_LDS uint32_t*)(mt + l32 * 32 + 8 * g + 4 * half);
      }
      // S = Q K^T and dP - D = dO V^T - D: A operands Q, dO rows l32 at d = 16 ds + 8 half, B operand
      // K from LDS (row 32 wave + l32); fragments read one k-step ahead
      f32x16 s = zero16();
      f32x16 dp;
      {
        const FA_LDS float* nd = (const FA_LDS float*)(st + 2 * QTILE) + 64 + 4 * half;
        const f32x4 a = *(const FA_LDS f32x4*)(nd), b4 = *(const FA_LDS f32x4*)(nd + 8);
        const f32x4 c = *(const FA_LDS f32x4*)(nd + 16), d4 = *(const FA_LDS f32x4*)(nd + 24);
        dp = __builtin_shufflevector(__builtin_shufflevector(a, b4, 0, 1, 2, 3, 4, 5, 6, 7),
                                     __builtin_shufflevector(c, d4, 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2, 3, 4, 5, 6, 7, 8,
                                     9, 10, 11, 12, 13, 14, 15);
        if constexpr (DROP) dp *= (float)dr.t * (1.f / 256.f);
      }
      bf16x8 fq[2], fd[2], fk[2];
      auto rd = [&](int ds) {
        const uint32_t off = tile_off<D>(l32, 16 * ds + 8 * half);
        fq[ds & 1] = lds_read_b128(st, off);
        fd[ds & 1] = lds_read_b128(st + QTILE, off);
        fk[ds & 1] = lds_read_b128(kst, tile_off<D>(32 * wave + l32, 16 * ds + 8 * half));
      };
      rd(0);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        __builtin_amdgcn_sched_barrier(0);
        if (ds + 1 < DS) rd(ds + 1);
        s = mfma32x32x16(fq[ds & 1], fk[ds & 1], s);
        dp = mfma32x32x16(fd[ds & 1], vb[ds], dp);
      }
      __builtin_amdgcn_sched_barrier(0);

      // P = exp2(S c - LSE log2 e) (hidden pairs 0), dS = P (dP - D); element r holds query
      // 8 (r / 4) + 4 half + r % 4 of the tile
      float cf = c_log2;
      if ((bool)mask) {
        const int qi0 = (it0 + u) * kBrKl;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int query = qi0 + 8 * (r >> 2) + 4 * half + (r & 3);
          s[r] = (my_key <= query) ? s[r] * c_log2 : -INFINITY;
        }
        cf = 1.f;
      }
      const FA_LDS float* lse_t = (const FA_LDS float*)(st + 2 * QTILE);
      f32x4 l4[4], nd4[DROP ? 4 : 1];
#pragma unroll
      for (int gq = 0; gq < 2; ++gq) {
        l4[gq] = *(const FA_LDS f32x4*)(lse_t + 8 * gq + 4 * half);
        if constexpr (DROP) nd4[gq] = *(const FA_LDS f32x4*)(lse_t + 64 + 8 * gq + 4 * half);
      }
      auto unit = [&](int r) {
        const float pr_ = fast_exp2(fmaf(s[r], cf, -l4[r >> 2][r & 3]));
        float dpv = dp[r];  // dP - D (dropout: dP - D t / 256)
        float pv = pr_;     // P for dV: the kept probabilities (their 256/t scale is applied to dV at the end)
        if constexpr (DROP) {
          const bool keep = dropout_keep(dr, kwt[r >> 2], r & 3);
          dpv = keep ? dpv * dr.scale : nd4[r >> 2][r & 3];  // (256 / t) dP - D, or 0 - D
          pv = keep ? pr_ : 0.f;
        }
        dp[r] = pr_ * dpv;
        s[r] = pv;
      };
      // the first query half (elements 0..7) before the dV/dK products; the second beside the first
      // half's products, which do not need it
#pragma unroll
      for (int r = 0; r < 8; ++r) unit(r);
      const bf16x8 pb0 = pack8(s, 0), db0 = pack8(dp, 0);
      bf16x8 pb1, db1;

      // dV^T += dO^T P, dK^T += Q^T dS: (ks, dt) steps, query half ks outermost; A operands through
      // the transposing read, one step ahead
      bf16x8 bd[2], bq[2];
      auto rdb = [&](int i) {
        const int ks = i / DT, dt = i % DT;
        const uint32_t tb0 = tile_off<D>(trow, 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3)) + ks * 16 * D * 2;
        const uint32_t tb8 = tile_off<D>(trow + 8, 32 * dt + 16 * (g16 & 1) + 4 * (j16 & 3)) + ks * 16 * D * 2;
        bd[i & 1] = cat(lds_read_tr(st + QTILE, tb0), lds_read_tr(st + QTILE, tb8));
        bq[i & 1] = cat(lds_read_tr(st, tb0), lds_read_tr(st, tb8));
      };
      rdb(0);
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < 2 * DT) rdb(i + 1);
        const int dt = i % DT;
        dvt[dt] = mfma32x32x16(bd[i & 1], i < DT ? pb0 : pb1, dvt[dt]);
        dkt[dt] = mfma32x32x16(bq[i & 1], i < DT ? db0 : db1, dkt[dt]);
        if (i == 0) {  // (read here rather than above, which would not fit the registers)
          l4[2] = *(const FA_LDS f32x4*)(lse_t + 16 + 4 * half);
          l4[3] = *(const FA_LDS f32x4*)(lse_t + 24 + 4 * half);
        }
        if constexpr (DROP) {  // -D of the second half, each group read just before its elements
          if (i == 0) nd4[2] = *(const FA_LDS f32x4*)(lse_t + 64 + 16 + 4 * half);
          if (i == 2) nd4[3] = *(const FA_LDS f32x4*)(lse_t + 64 + 24 + 4 * half);
        }
        if (i < DT) {  // elements 8..15, two per step of the first half
          unit(8 + 2 * i);
          unit(9 + 2 * i);
          if (i == DT - 1) {
            pb1 = pack8(s, 8);
            db1 = pack8(dp, 8);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    FA_LDS char* const st[4] = {(FA_LDS char*)st0_raw, (FA_LDS char*)st1_raw, (FA_LDS char*)st2_raw,
                                (FA_LDS char*)st3_raw};
    // Tile u lives in stage u % 4.  Before tile u: tile u must have landed (tiles u+1, u+2 may still be
    // in flight); after the barrier every wave is done with tile u-1, whose stage receives tile u+3.
    // Every wave runs every tile (one barrier each); its form is chosen per wave.
    auto at = [&](auto stg, int u, int form) __attribute__((always_inline)) {
      constexpr int S = decltype(stg)::value;
      if (u + 2 < count) wait_vmem_n<2 * VPT>();
      else if (u + 1 < count) wait_vmem_n<VPT>();
      else wait_vmem();
      barrier();
      if (u + 3 < count) load_tile(u + 3, st[(S + 3) & 3]);
      if (form == 1) step(std::true_type{}, st[S], u);
      else if (form == 2) step(std::false_type{}, st[S], u);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // form of tile u for this wave: 0 none, 1 masked, 2 clean
    auto form_of = [&](int u) { return !CAUSAL ? 2 : u < tskip ? 0 : u < tskip + 4 ? 1 : 2; };

    load_tile(0, st[0]);
    if (count > 1) load_tile(1, st[1]);
    if (count > 2) load_tile(2, st[2]);
    wait_vmem_n<0>();  // (K rows too)
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) pin(vb[ds]);
    int u = 0;
    if constexpr (CAUSAL) {
      // the first 8 tiles: per-wave forms, stages picked at run time
      const int nh = min(count, 8);
#pragma nounroll
      for (; u < nh; ++u) {
        const int sidx = u & 3;
        FA_LDS char* const sc = sidx == 0 ? st[0] : sidx == 1 ? st[1] : sidx == 2 ? st[2] : st[3];
        FA_LDS char* const sl = sidx == 0 ? st[3] : sidx == 1 ? st[0] : sidx == 2 ? st[1] : st[2];
        if (u + 2 < count) wait_vmem_n<2 * VPT>();
        else if (u + 1 < count) wait_vmem_n<VPT>();
        else wait_vmem();
        barrier();
        if (u + 3 < count) load_tile(u + 3, sl);
        const int form = form_of(u);
        if (form != 0) step(form == 1, sc, u);
      }
    }
    // fully visible tiles, four per iteration so that the stages stay compile-time
    for (; u + 3 < count; u += 4) {
      at(I0{}, u, 2);
      at(I1{}, u + 1, 2);
      at(I2{}, u + 2, 2);
      at(I3{}, u + 3, 2);
    }
    if (u < count) at(I0{}, u, 2);
    if (u + 1 < count) at(I1{}, u + 1, 2);
    if (u + 2 < count) at(I2{}, u + 2, 2);
  }

  // ---- dK = scale dS^T Q, dV: lane holds key my_key, d = 32 dt + 8 gq + 4 half + 0..3.  Keys at or
  // past the valid length get zero gradients.  Each wave stages its 32 rows of dK and dV in LDS (16 KiB:
  // waves 0-3 in the K area, waves 4-7 in one ring stage each) and writes them back as whole 16-byte
  // chunks.
  constexpr int VB = kKeysKl * D * 2;  // bytes of the wave's dK rows (dV rows follow)
  static_assert(4 * 2 * VB <= kBcKl * D * 2 && 2 * VB <= STAGE, "the staging areas hold a wave's rows");
  barrier();  // every wave is done with K and the query tiles
  {
    FA_LDS char* const ep = wave < 4 ? (FA_LDS char*)kst_raw + wave * 2 * VB
                            : wave == 4 ? (FA_LDS char*)st0_raw
                            : wave == 5 ? (FA_LDS char*)st1_raw
                            : wave == 6 ? (FA_LDS char*)st2_raw : (FA_LDS char*)st3_raw;
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
    constexpr int CHUNKS = kKeysKl * (D / 8) / 64;  // 16-byte chunks per lane and tensor
#pragma unroll
    for (int n = 0; n < CHUNKS; ++n) {
      const int pch = n * 64 + lane;
      const int r = pch / (D / 8), c = pch % (D / 8);
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

template <bool CAUSAL, bool PADDED, bool DROP>
hipError_t launch_kl(const Problem& p, const void* q, const void* k, const void* v, const void* dO, const float* lse2,
                     const float* ndelta, void* dk, void* dv) {
  const int nkb = (p.N + kBcKl - 1) / kBcKl;
  const int BH = p.B * p.H;
  const Dropout dr{p.drop_k0, p.drop_k1, p.drop_off2, p.drop_t, 256.f / (float)p.drop_t};
  hipLaunchKernelGGL((bwd_dkdv_kl_kernel<CAUSAL, PADDED, DROP>), dim3((unsigned)(nkb * BH)), dim3(kWkl * 64), 0,
                     p.stream, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO, lse2, ndelta,
                     (__bf16*)dk, (__bf16*)dv, p.H, p.N, p.scale, p.scale * kLog2e, p.seqlens, dr, BH);
  return hipGetLastError();
}

template <bool DROP>
hipError_t launch_kl_m(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                       const float* lse2, const float* ndelta, void* dk, void* dv) {
  const bool pad = p.seqlens != nullptr;
  if (p.causal)
    return pad ? launch_kl<true, true, DROP>(p, q, k, v, dO, lse2, ndelta, dk, dv)
               : launch_kl<true, false, DROP>(p, q, k, v, dO, lse2, ndelta, dk, dv);
  return pad ? launch_kl<false, true, DROP>(p, q, k, v, dO, lse2, ndelta, dk, dv)
             : launch_kl<false, false, DROP>(p, q, k, v, dO, lse2, ndelta, dk, dv);
}

}  // namespace

hipError_t launch_dkdv_kl_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* dO,
                               const float* lse2, const float* ndelta, void* dk, void* dv) {
  return p.dropout ? launch_kl_m<true>(p, q, k, v, dO, lse2, ndelta, dk, dv)
                   : launch_kl_m<false>(p, q, k, v, dO, lse2, ndelta, dk, dv);
}

}  // namespace fa
