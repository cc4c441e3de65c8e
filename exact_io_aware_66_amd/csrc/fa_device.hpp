// Device-side building blocks shared by the gfx950 attention kernels.
//
// Everything here is specific to CDNA4 (gfx950): wave64, the bf16 matrix-core instruction
// v_mfma_f32_32x32x16_bf16, the transposing LDS read ds_read_b64_tr_b16 and the direct
// global->LDS loads (global_load_lds_dwordx4, buffer_load_dwordx4 ... lds).
//
// Lane layouts used by the kernels (wave64, lane l, half h = l / 32):
//   32x32x16 MFMA  A[32][16]: lane l holds row l%32, k = 8h .. 8h+7
//                  B[16][32]: lane l holds column l%32, k = 8h .. 8h+7
//                  C[32][32]: lane l holds column l%32, rows 8(r/4) + 4h + r%4 for r = 0..15
//   ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element i%4 of the 8-byte rows
//                  addressed by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of its group.
//   global_load_lds_dwordx4 / buffer_load_dwordx4 lds: lane i of a wave writes its 16 bytes at
//                  LDS base + 16 i (the base is wave-uniform, passed in M0).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));  // 32 FP8 values: an operand of the FP8 MFMA

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// XOR swizzle of the 16-byte chunk index inside one row of a row-major bf16 LDS tile with NCOL
// columns, keyed by the row.  gfx950's LDS serves a transposing 64-bit read 32 lanes (256 bytes, 64
// banks) at a time; in our reads those lanes cover 4 consecutive rows (aligned to 4) x 4 aligned
// chunks, so the 4 rows must land on disjoint bank ranges.  128-bit reads of 16 consecutive rows at
// one logical chunk must land on distinct chunk positions too.
//   256-byte rows (NCOL = 128): s(r) = 4 (r mod 4) + (r / 4 mod 4)
//   128-byte rows (NCOL = 64):  s(r) = 4 (r / 2 mod 2) + (r / 4 mod 4)   (two rows share a bank range)
// In both, s(r + 16) = s(r) and s(r + 8) = s(r) xor 2.
template <int NCOL>
__device__ __forceinline__ int swz(int row) {
  static_assert(NCOL == 64 || NCOL == 128, "swizzle defined for 128- and 256-byte rows");
  return NCOL == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Byte offset of (row, element col) in a row-major LDS tile of NCOL bf16 per row, swizzled.
template <int NCOL>
__device__ __forceinline__ uint32_t tile_off(int row, int col) {
  const int c = col >> 3;
  return (uint32_t)(row * (NCOL * 2) + ((c ^ swz<NCOL>(row)) << 4) + ((col & 7) << 1));
}

// Software-pipelined schedule for STEPS steps of (R LDS reads -> M MFMAs [+ V VALU]): the reads
// run AHEAD steps in front of the MFMAs that consume them, so LDS latency overlaps matrix work.
// Applies to the instructions of the current scheduling region (sync id SYNC).
template <int STEPS, int R, int M, int V, int AHEAD, int SYNC>
__device__ __forceinline__ void pipe_schedule() {
#pragma unroll
  for (int i = 0; i < AHEAD && i < STEPS; ++i) __builtin_amdgcn_sched_group_barrier(0x100, R, SYNC);
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, SYNC);
      if (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, SYNC);
    }
    if (i + AHEAD < STEPS) __builtin_amdgcn_sched_group_barrier(0x100, R, SYNC);
  }
}

__device__ __forceinline__ bf16x8 lds_read_b128(const FA_LDS char* base, uint32_t off) {
  return *(const FA_LDS bf16x8*)(base + off);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const FA_LDS char* base, uint32_t off) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(base + off));
  return __builtin_bit_cast(bf16x4, v);
}

// The same transposing read issued through inline assembly.  The compiler then does not treat it as
// an LDS load that may alias an in-flight direct global->LDS prefetch (for the builtin it inserts a
// full vmcnt wait, serialising the prefetch); the caller must wait for the result with
// lds_wait() before using it.  `addr` is the byte address inside LDS.
template <int OFFSET = 0>
__device__ __forceinline__ u32x2 lds_read_tr_asm(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFFSET));
  return r;
}

// Wait for every outstanding LDS access of this wave; the listed values become dependent on the
// wait so their uses cannot be scheduled above it.
__device__ __forceinline__ void lds_wait(u32x2& a, u32x2& b) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b)); }
__device__ __forceinline__ void lds_wait(u32x2& a, u32x2& b, u32x2& c, u32x2& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void lds_wait(u32x2& a, u32x2& b, u32x2& c, u32x2& d, u32x2& e, u32x2& f, u32x2& g,
                                         u32x2& h) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d), "+v"(e), "+v"(f), "+v"(g), "+v"(h));
}

__device__ __forceinline__ uint32_t lds_addr(const FA_LDS void* p) { return (uint32_t)(uintptr_t)p; }

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 cat(u32x2 a, u32x2 b) {
  return cat(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b));
}

// 16 bytes from global memory straight into LDS at (wave-uniform) lds_base + 16 * lane.
__device__ __forceinline__ void gload_lds16(const void* gptr, FA_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 16, 0, 0);
}
// 4 bytes from global memory into LDS at (wave-uniform) lds_base + 4 * lane.
__device__ __forceinline__ void gload_lds4(const void* gptr, FA_LDS void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 4, 0, 0);
}

// Buffer resource (4 SGPRs) over `bytes` bytes from a wave-uniform base: raw addressing, stride 0.
// A buffer load whose per-lane byte offset is >= bytes returns zeros instead of touching memory, so
// rows past the end of a tensor need neither a clamp nor a branch.  The fourth word is the
// gfx9-family raw-buffer format.
// (The fields go through readfirstlane, as does the LDS base of the loads below: they are
// wave-uniform, and the inline assembly that uses them requires scalar registers.)
__device__ __forceinline__ u32x4 make_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu),
               (uint32_t)__builtin_amdgcn_readfirstlane(max(bytes, 0)), 0x00020000u};
}
// 16 bytes at byte offset voff of the buffer straight into LDS at (wave-uniform) lds_base + 16 * lane
// (buffer_load_dwordx4 ... lds, LDS base in M0).  Issued through inline assembly so that the
// compiler does not track the asynchronous LDS write: it would otherwise wait for every
// outstanding load (vmcnt(0)) before reads of an unrelated LDS stage.  The caller orders the
// transfer with wait_vmem / wait_vmem_n and a barrier before any wave reads the destination.
//
// FA_POISON_LDS (a debug build, libfa_poison.so): each lane first fills its own destination bytes
// with all-ones words (NaN in bf16, fp32 and FP8 E4M3) and waits for that store, so that a wave
// reading a stage before the transfer has landed, or after the stage was handed to the next tile,
// reads NaN instead of plausible stale data; correctly synchronised kernels give results bitwise
// equal to the release build.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is reserved: no compiler-generated code here relies on it
__device__ __forceinline__ void poison_lds(const FA_LDS void* lds_base, int bytes_per_lane) {
#ifdef FA_POISON_LDS
  FA_LDS char* const p = (FA_LDS char*)const_cast<FA_LDS void*>(lds_base) + bytes_per_lane * (threadIdx.x & 63);
  if (bytes_per_lane == 16) *(volatile FA_LDS u32x4*)p = u32x4{~0u, ~0u, ~0u, ~0u};
  else *(volatile FA_LDS uint32_t*)p = ~0u;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#else
  (void)lds_base;
  (void)bytes_per_lane;
#endif
}
// The work item of this workgroup: its id in the grid, or (FA_POISON_LDS debug build) the ids in
// reverse order, so that every item runs on other compute units, in another order and beside other
// items than in the release build; each output element has one writer and a fixed summation order,
// so the results must not change.
__device__ __forceinline__ int work_item() {
#ifdef FA_POISON_LDS
  return (int)(gridDim.x - 1 - blockIdx.x);
#else
  return (int)blockIdx.x;
#endif
}
__device__ __forceinline__ void bload_lds16(u32x4 r, uint32_t voff, const FA_LDS void* lds_base) {
  poison_lds(lds_base, 16);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base))
               : "memory", "m0");
}
// 4 bytes at byte offset voff of the buffer into LDS at (wave-uniform) lds_base + 4 * lane.
__device__ __forceinline__ void bload_lds4(u32x4 r, uint32_t voff, const FA_LDS void* lds_base) {
  poison_lds(lds_base, 4);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base))
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N vector-memory instructions of this wave are outstanding (they complete in
// issue order for loads), i.e. everything but the last N issued has landed.
template <int N>
__device__ __forceinline__ void wait_vmem_n() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Workgroup barrier without the memory fence of __syncthreads().  The fence would make the
// compiler wait for every outstanding direct-to-LDS load (vmcnt(0)), including prefetches that are
// meant to stay in flight across the barrier.  Callers first wait (vmcnt) for the loads whose data
// other waves read after the barrier.  The memory clobber keeps every LDS access of the wave on
// its side of the barrier; the LDS reads issued before it have all been consumed (and so have
// completed) by then, so no lgkmcnt wait is needed for the stage that is reloaded after it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
// The same barrier once this wave's LDS stores have completed (lgkmcnt(0)): for tiles that the
// waves write into LDS themselves.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Keeps the computation of x where it stands: the (empty) volatile statement consumes and
// redefines x, so the code that produces x is not moved past later volatile statements (barriers).
template <class T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// Value of x in lane l ^ 32 combined with x by max / add (one v_permlane32_swap).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float min_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 8 consecutive fp32 accumulator values -> 8 bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  f32x2 a = {s[base + 0], s[base + 1]}, b = {s[base + 2], s[base + 3]};
  f32x2 c = {s[base + 4], s[base + 5]}, d = {s[base + 6], s[base + 7]};
  bf16x2 pa = __builtin_convertvector(a, bf16x2), pb = __builtin_convertvector(b, bf16x2);
  bf16x2 pc = __builtin_convertvector(c, bf16x2), pd = __builtin_convertvector(d, bf16x2);
  bf16x4 lo = __builtin_shufflevector(pa, pb, 0, 1, 2, 3);
  bf16x4 hi = __builtin_shufflevector(pc, pd, 0, 1, 2, 3);
  return cat(lo, hi);
}

// 8 consecutive floats of an array -> 8 bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack8f(const float* v, int base) {
  f32x2 a = {v[base + 0], v[base + 1]}, b = {v[base + 2], v[base + 3]};
  f32x2 c = {v[base + 4], v[base + 5]}, d = {v[base + 6], v[base + 7]};
  bf16x2 pa = __builtin_convertvector(a, bf16x2), pb = __builtin_convertvector(b, bf16x2);
  bf16x2 pc = __builtin_convertvector(c, bf16x2), pd = __builtin_convertvector(d, bf16x2);
  return cat(__builtin_shufflevector(pa, pb, 0, 1, 2, 3), __builtin_shufflevector(pc, pd, 0, 1, 2, 3));
}

__device__ __forceinline__ bf16x4 pack4(float a0, float a1, float a2, float a3) {
  f32x2 a = {a0, a1}, b = {a2, a3};
  bf16x2 pa = __builtin_convertvector(a, bf16x2), pb = __builtin_convertvector(b, bf16x2);
  return __builtin_shufflevector(pa, pb, 0, 1, 2, 3);
}

__device__ __forceinline__ int clamp_len(const int32_t* seqlens, int b, int N) {
  int L = seqlens[b];
  return L < 0 ? 0 : (L > N ? N : L);
}

// ---- dropout: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
// 1, 2, 3", SC'11) and the keep decision of one (query, key) element.
//
// Element (bh, query i, key j) draws the byte of key j % 32 = 8 g + 4 h + e from output word g,
// byte e, of Philox4x32-10 with counter (i, j / 32, bh, 2 offset + h) and key (seed low, seed high);
// it is kept when that byte is below t = round((1 - p) 256), and kept probabilities are scaled by
// 256 / t.  A lane that holds one query and the 16 keys 8 g + 4 h + e of a 32-key block (the score
// layout of the forward and dQ kernels) needs exactly one call per block.
struct Dropout {
  uint32_t k0, k1;  // seed, low and high words
  uint32_t off2;    // 2 offset
  uint32_t t;       // keep threshold, 1..256
  float scale;      // 256 / t
};

// a ^ b ^ k in one instruction (v_bitop3_b32, truth table 0x96 = three-input XOR; the compiler emits
// two v_xor_b32 for it); k is wave-uniform (a scalar register written by scalar instructions)
__device__ __forceinline__ uint32_t xor3_vvs(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

// X3: the three-input XORs as single instructions (fewer instructions, but an opaque statement the
// register allocator cannot move; used where registers are not the limit)
template <bool X3 = false>
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t n0 = X3 ? xor3_vvs((uint32_t)(p1 >> 32), c1, k0) : (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = X3 ? xor3_vvs((uint32_t)(p0 >> 32), c3, k1) : (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// The four keep words of (query i, 32-key block jb, half h): byte e of word g is key 8 g + 4 h + e.
template <bool X3 = false>
__device__ __forceinline__ u32x4 dropout_words(const Dropout& dr, uint32_t bh, int i, int jb, int h) {
  return philox4x32_10<X3>((uint32_t)i, (uint32_t)jb, bh, dr.off2 + (uint32_t)h, dr.k0, dr.k1);
}

__device__ __forceinline__ bool dropout_keep(const Dropout& dr, uint32_t word, int e) {
  return ((word >> (8 * e)) & 0xFFu) < dr.t;
}

// ---- block-sparse attention: the visible tiles of a workgroup, compacted into an LDS list
//
// The block mask has 128 x 128 blocks; a kernel tile (a run of keys or of queries) never straddles
// two blocks.  For a run of blocks [b0, b1) of one mask row or column, flags(b) is nonzero when block
// b is visible (its low bits may carry per-wave visibility), and each visible block contributes its
// tiles [b TPB, min((b + 1) TPB, tile_end)), b1 = ceil(tile_end / TPB).  Entries are
// tile | flags << 12, in increasing tile order; the tile count goes to *count.  One whole wave runs
// it; the caller synchronises before the list is read.
constexpr int kMaskBlock = 128;       // rows and columns of one mask block
constexpr int kMaxMaskBlocks = 1024;  // blocks per side of the largest block mask (N <= 131072)
constexpr int kTileBits = 12;         // tile index bits of a list entry

template <int TPB, class Flags>
__device__ __forceinline__ void compact_tiles(FA_LDS uint16_t* list, FA_LDS int* count, int b0, int b1, int tile_end,
                                              Flags flags) {
  const int lane = threadIdx.x & 63;
  int total = 0;  // visible blocks so far (wave-uniform)
  for (int c = b0; c < b1; c += 64) {
    const int blk = c + lane;
    const int f = blk < b1 ? flags(blk) : 0;
    const uint64_t m = __ballot(f != 0);
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (f != 0) {
#pragma unroll
      for (int i = 0; i < TPB; ++i) {
        const int tile = blk * TPB + i;
        if (tile < tile_end) list[(total + rank) * TPB + i] = (uint16_t)(tile | (f << kTileBits));
      }
    }
    total += __popcll(m);
  }
  const int last = b1 > b0 ? flags(b1 - 1) : 0;  // the last block may hold fewer than TPB tiles
  if (lane == 0) *count = total * TPB - (last != 0 ? b1 * TPB - tile_end : 0);
}

__device__ __forceinline__ int list_tile(uint16_t e) { return e & ((1 << kTileBits) - 1); }
__device__ __forceinline__ int list_flags(uint16_t e) { return e >> kTileBits; }

// Number of list entries whose tile is below x (the list is sorted by tile).
__device__ __forceinline__ int count_below(const FA_LDS uint16_t* list, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (list_tile(list[mid]) < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

}  // namespace fa
