// Grouped expert GEMMs on CDNA4 matrix cores.
//
// LLM Internals 14.2.1 step 5: every expert multiplies its own m_i rows,
// [m_i, d] x W_i[d, F] -> [m_i, F], then projects back to d; the row counts
// differ per expert.  One expert is a SwiGLU block of three matrices
// (14.2.2): h = silu(x W1) * (x W3), y = h W2.
//
// Kernel shape (one launch per projection):
//   * a device-built work list holds one entry per (expert, M-tile, N-tile),
//     or per K part of the down projection's tiles that follow its last full
//     dispatch round; it is ordered expert by expert, and inside an expert in
//     groups of up to 8 M-tiles, runs of NG neighbouring N-tiles and the
//     M-tiles fastest, so the tiles that run at the same time on one XCD
//     share both their weight slices and their activation rows in that
//     XCD's L2;
//   * one block per list entry, one block per CU at a time; blocks are
//     mapped to entries so that in each round of (CUs) blocks every XCD
//     works on a contiguous run of the list;
//   * block tile BM x BNT with four waves of (BM/WM) x (BNT/WN); the large
//     configuration gives each wave 128 x 128 outputs: 16 MFMA blocks of
//     32x32 per 8 fragment loads, accumulators in AGPRs, one wave per SIMD;
//   * three kernels share the tile logic.  k_moe_gemm_dma (medium tiles,
//     FP8 decode tiles) copies each stage from global memory straight
//     into LDS rings (global_load_lds), described at the kernel.
//     k_moe_gemm (bf16 decode, fp32) stages through registers: BK = 128
//     bytes of K per stage, two LDS stages and two register staging sets,
//     stage k+2 fetched while stage k+1 is stored to LDS.  k_moe_pp (both
//     projections of the large tiles, bf16 or FP8 weights) runs eight waves as two groups
//     that alternate memory and compute phases (ping-pong);
//   * in both, a software pipeline over k16 substeps reads each substep's
//     fragments while the previous substep's MFMAs run; scheduling groups
//     pin the interleave;
//   * LDS rows are 8 chunks of 16 B, chunk c of row r at slot
//     c ^ ((r ^ (r/8 mod 4)) mod 8): the 16-B stores and the fragment reads
//     are bank-conflict free whether the LDS serves 8 or 16 lanes per cycle;
//   * a wave skips the MFMAs of its 32-row blocks that lie past the tile's
//     last row (a ragged last M-tile of an expert computes only live rows);
//   * bf16: v_mfma_f32_32x32x16_bf16 in the four-wave kernels and
//     v_mfma_f32_16x16x32_bf16 in k_moe_pp, each lane feeding 8 K-contiguous
//     values per operand; fp32: four v_mfma_f32_32x32x2f32 per 16-B fragment;
//   * gate/up fusion: the B tile holds BN rows of W1 then BN rows of W3, a
//     wave owns matching gate and up columns, and SwiGLU runs on the fp32
//     accumulators before one rounding of h to the storage type;
//   * epilogues: bf16 h is stored from the accumulators (8 bytes per lane);
//     the down projection's fp32 rows pass through LDS so that each store
//     instruction writes whole lines (store_tile_staged).
#include <cmath>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace moe {

template <typename T>
__device__ __forceinline__ void mma_32x32(f32x16& acc, const u32x4& a, const u32x4& b) {
  if constexpr (sizeof(T) == 2) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), acc,
                                                 0, 0, 0);
  }
}

// silu(x) = x sigmoid(x) in fp32: hardware exp and reciprocal (about 1 ulp
// each), far below the one rounding of h to bf16 that follows.
__device__ __forceinline__ float silu_f(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}


constexpr int kThreads = 256;   // four waves per block

// One K stage, global -> registers.  Thread t owns the 16-B chunk t%8 of
// rows t/8, t/8 + 32, ... of the A tile and of the B tile.
template <typename T, int CA, int CB, bool GLU, int BN>
__device__ __forceinline__ void gload_tile(u32x4 (&ra)[CA], u32x4 (&rb)[CB],
                                           const T* const (&pa)[CA], const T* pb0,
                                           const T* pb1, size_t bstep, int k0) {
#pragma unroll
  for (int i = 0; i < CA; ++i) ra[i] = *(const u32x4*)(pa[i] + k0);
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    constexpr int kSplit = BN / (kThreads / 8);   // first thread-row index in the W3 half
    const T* p = (GLU && i >= kSplit) ? pb1 + (size_t)(i - kSplit) * bstep
                                      : pb0 + (size_t)i * bstep;
    rb[i] = *(const u32x4*)(p + k0);
  }
}

// LDS swizzle: chunk c of row r is stored at slot c ^ swz(r).  swz depends on
// r mod 32 only, and is a bijection on any 8 rows starting at a multiple of
// 8 and on the even and on the odd rows of any 16 rows starting at a
// multiple of 16, so 16-B accesses by 8 lanes on 8 rows or by 16 lanes on 16
// rows (one chunk column), and by 8 or 16 lanes covering whole rows, all hit
// distinct banks.
__device__ __forceinline__ int swz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

// K stage that the loop's stage x reads: x + rot taken modulo nk (x, rot < nk).
__device__ __forceinline__ int kstage(int x, int rot, int nk) {
  return x + rot >= nk ? x + rot - nk : x + rot;
}

// Height of the M-tiles of a group of n rows: ceil(n / BM) tiles of equal
// height rounded up to whole 32-row blocks (the last tile takes the rest).
// A group slightly larger than a multiple of BM then gets a few slightly
// shorter tiles instead of full tiles plus one of a handful of rows, which
// would cost nearly a full tile's copies.  Every tile holds at least one
// row: n > (ceil(n / BM) - 1) BM >= (ceil(n / BM) - 1) height.
__host__ __device__ __forceinline__ int tile_height(int n, int BM) {
  if (n <= BM) return BM;
  const int mt = (n + BM - 1) / BM;
  const int h = ((n + mt - 1) / mt + 31) & ~31;
  return h < BM ? h : BM;
}

// Registers -> one LDS stage.  Rows r and r + 32 i share swz(r).
template <int BM, int CA, int CB>
__device__ __forceinline__ void lstore_tile(u32x4* sm, const u32x4 (&ra)[CA],
                                            const u32x4 (&rb)[CB], int tid) {
  const int r0 = tid >> 3;
  const int c = (tid & 7) ^ swz(r0);
#pragma unroll
  for (int i = 0; i < CA; ++i) sm[(r0 + i * (kThreads / 8)) * 8 + c] = ra[i];
#pragma unroll
  for (int i = 0; i < CB; ++i) sm[(BM + r0 + i * (kThreads / 8)) * 8 + c] = rb[i];
}

// Fragments of one k16 substep.  A lane's fragment rows are all congruent
// to lane % 32 modulo 32, so they share swz(row) and one swizzled chunk index
// per substep (cs) serves every fragment: A rows are pa + 32 i rows, B rows
// pb + the wave's column rows.
template <int NA, int FM, int FN, int BN, bool GLU>
__device__ __forceinline__ void load_frags(u32x4* f, const u32x4* pa, const u32x4* pb, int cs) {
  constexpr int FNH = GLU ? FN / 2 : FN;
#pragma unroll
  for (int i = 0; i < NA; ++i) f[i] = pa[i * 32 * 8 + cs];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int rr = GLU ? ((j < FNH) ? j * 32 : BN + (j - FNH) * 32) : j * 32;
    f[FM + j] = pb[rr * 8 + cs];
  }
}

// MFMAs of one substep for the first NV 32-row blocks of the wave's tile.
// The weight fragment is the MFMA's first operand, so each accumulator holds
// a transposed 32x32 block: lane & 31 selects the token row, and element
// 4q + e (q, e < 4) the output column 8q + 4 (lane >> 5) + e, i.e. every
// lane owns runs of four consecutive outputs of one row.
template <typename T, int NV, int FM, int FN>
__device__ __forceinline__ void mma_substep(f32x16 (&acc)[FM][FN], const u32x4* f) {
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) mma_32x32<T>(acc[i][j], f[FM + j], f[i]);
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100,
              kSchedDsWrite = 0x200;

// Scheduling groups for one MFMA substep: NM MFMAs with ND fragment reads,
// then NG global loads, then NW LDS stores threaded between them one per
// MFMA; what does not fit follows.
template <int NM, int ND, int NG, int NW>
__device__ __forceinline__ void sched_substep() {
  constexpr int P1 = ND < NM ? ND : NM;
  constexpr int R1 = NM - P1;
  constexpr int P2 = NG < R1 ? NG : R1;
  constexpr int R2 = R1 - P2;
  constexpr int P3 = NW < R2 ? NW : R2;
  constexpr int R3 = R2 - P3;
#pragma unroll
  for (int i = 0; i < P1; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  if constexpr (ND - P1 > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, ND - P1, 0);
#pragma unroll
  for (int i = 0; i < P2; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
  }
  if constexpr (NG - P2 > 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, NG - P2, 0);
#pragma unroll
  for (int i = 0; i < P3; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
  }
  if constexpr (NW - P3 > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, NW - P3, 0);
  if constexpr (R3 > 0) __builtin_amdgcn_sched_group_barrier(kSchedMfma, R3, 0);
}

// Main K loop of one tile for a wave whose first NV (of FM) 32-row blocks
// hold real rows; blocks past the tile's last row skip their MFMAs and
// fragment reads (NV = 0: the wave only loads and stores its share of the
// stages).  Every wave runs the same loads, stores and barriers.
//
// Software pipeline over k16 substeps with two fragment slots and two
// register staging sets.  Iteration kt (stage kt in LDS buffer kt&1):
//   issue global loads of stage kt+2 into staging set (kt+1)&1
//   MFMA stage kt-1 substep 3 (slot 1)  | read stage kt substep 0 (slot 0)
//   MFMA substep 0 (slot 0)             | read substep 1 (slot 1)
//   MFMA substep 1 (slot 1)             | read substep 2 (slot 0),
//                                          store staging set kt&1 (stage
//                                          kt+1) to LDS buffer (kt+1)&1
//   MFMA substep 2 (slot 0)             | read substep 3 (slot 1)
//   barrier
// so every global load has about 1.6 stages to arrive.  Loop stage kt reads
// K stage (kt + rot) mod nk.  Loads past the last stage re-fetch the last
// stage (in bounds, never used).  Slot 1 starts as
// zeros: the first iteration's leading MFMAs add 0.  nk is even (K is a
// multiple of 128 elements), so the loop advances two stages at a time and
// the staging sets keep fixed names.
template <typename T, int NV, int BM, int BN, int CA, int CB, int FM, int FN, bool GLU>
__device__ __forceinline__ void main_loop(f32x16 (&acc)[FM][FN], u32x4 (*smem)[1],
                                          const T* const (&oa)[CA], const T* pb0, const T* pb1,
                                          size_t bstep, int nk, int fa, int fb,
                                          const int (&cs)[4], int tid, int rot) {
  constexpr int NF = FM + FN;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int BK = 8 * EPC;
  u32x4* sm0 = smem[0];
  u32x4* sm1 = sm0 + (BM + (GLU ? 2 * BN : BN)) * 8;
  u32x4 ra0[CA], rb0[CB], ra1[CA], rb1[CB];
  gload_tile<T, CA, CB, GLU, BN>(ra1, rb1, oa, pb0, pb1, bstep, kstage(0, rot, nk) * BK);
  gload_tile<T, CA, CB, GLU, BN>(ra0, rb0, oa, pb0, pb1, bstep,
                                 kstage(nk > 1 ? 1 : 0, rot, nk) * BK);
  lstore_tile<BM, CA, CB>(sm0, ra1, rb1, tid);
  __syncthreads();
  u32x4 f0[NF], f1[NF];
#pragma unroll
  for (int x = 0; x < NF; ++x) f1[x] = u32x4{0u, 0u, 0u, 0u};
  for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = kt + h;
      const u32x4* sm = h ? sm1 : sm0;
      const int kn = kstage(k + 2 < nk ? k + 2 : nk - 1, rot, nk) * BK;
      if (h == 0) gload_tile<T, CA, CB, GLU, BN>(ra1, rb1, oa, pb0, pb1, bstep, kn);
      else        gload_tile<T, CA, CB, GLU, BN>(ra0, rb0, oa, pb0, pb1, bstep, kn);
      if constexpr (NV > 0) {
        load_frags<NV, FM, FN, BN, GLU>(f0, sm + fa, sm + fb, cs[0]);
        mma_substep<T, NV, FM, FN>(acc, f1);
        load_frags<NV, FM, FN, BN, GLU>(f1, sm + fa, sm + fb, cs[1]);
        mma_substep<T, NV, FM, FN>(acc, f0);
        load_frags<NV, FM, FN, BN, GLU>(f0, sm + fa, sm + fb, cs[2]);
      }
      if (h == 0) lstore_tile<BM, CA, CB>(sm1, ra0, rb0, tid);
      else        lstore_tile<BM, CA, CB>(sm0, ra1, rb1, tid);
      if constexpr (NV > 0) {
        mma_substep<T, NV, FM, FN>(acc, f1);
        load_frags<NV, FM, FN, BN, GLU>(f1, sm + fa, sm + fb, cs[3]);
        mma_substep<T, NV, FM, FN>(acc, f0);
      }
      if constexpr (sizeof(T) == 2 && NV > 0) {
        constexpr int NM = NV * FN;
        constexpr int ND = NV + FN;
        constexpr int NL = CA + CB;
        sched_substep<NM, ND, NL / 2, 0>();
        sched_substep<NM, ND, NL - NL / 2, 0>();
        sched_substep<NM, ND, 0, NL>();
        sched_substep<NM, ND, 0, 0>();
      }
      __syncthreads();
    }
  }
  if constexpr (NV > 0) mma_substep<T, NV, FM, FN>(acc, f1);
}

// Tile epilogue.  Accumulator layout (see mma_substep): lane & 31 is the
// row inside a 32-row block, element 4q + e the column 8q + 4 (lane >> 5) + e
// of a 32-column block, so every lane stores runs of four consecutive
// outputs of its row: 8 bytes of bf16 h or 16 bytes of fp32 y per store.
// Rows past the tile's last row are masked per lane.
//   GLU : out = H (type T), h = silu(gate) * up rounded once
//   else: split 0 writes fp32 to out, split ks > 0 to slab ks - 1 of out2
// With SC (FP8 weights) the accumulators are first multiplied by the
// per-output-channel scales: gate by sc0[n], up by sc1[n], down by sc0[n].
template <typename T>
__device__ __forceinline__ void store4_h(T* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4_h<uint16_t>(uint16_t* p, float a, float b, float c,
                                                   float d) {
  *(uint2*)p = make_uint2(bf16x2_bits(a, b), bf16x2_bits(c, d));
}
template <>
__device__ __forceinline__ void store4_h<float>(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}

template <typename T, int BN, int BNT, int WN, int FM, int FN, bool GLU, bool SC = false>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[FM][FN], void* __restrict__ out,
                                           float* __restrict__ out2, int ks, int max_rows, int N,
                                           int rbeg, int rows, int arow0, int n0, int wn,
                                           int lane, const float* __restrict__ sc0 = nullptr,
                                           const float* __restrict__ sc1 = nullptr) {
  constexpr int FNH = GLU ? FN / 2 : FN;
  constexpr int WCOLS = BNT / WN;
  const int lr = arow0 + (lane & 31);                 // this lane's row in block 0
  const int cq = 4 * (lane >> 5);                     // column offset inside 8-column runs
  if constexpr (GLU) {
    const int cb = n0 + wn * (BN / WN) + cq;
    float4 sg[FNH][4], su[FNH][4];
#pragma unroll
    for (int j = 0; j < FNH; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sg[j][q] = SC ? *(const float4*)(sc0 + cb + j * 32 + 8 * q) : make_float4(1.f, 1.f, 1.f, 1.f);
        su[j][q] = SC ? *(const float4*)(sc1 + cb + j * 32 + 8 * q) : make_float4(1.f, 1.f, 1.f, 1.f);
      }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = lr + i * 32;
      if (row < rows) {
        T* H = (T*)out + (size_t)(rbeg + row) * N + cb;
#pragma unroll
        for (int j = 0; j < FNH; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& g = acc[i][j];
            const f32x16& u = acc[i][j + FNH];
            const float4 a = sg[j][q], b = su[j][q];
            store4_h<T>(H + j * 32 + 8 * q,
                        silu_f(g[4 * q] * a.x) * (u[4 * q] * b.x),
                        silu_f(g[4 * q + 1] * a.y) * (u[4 * q + 1] * b.y),
                        silu_f(g[4 * q + 2] * a.z) * (u[4 * q + 2] * b.z),
                        silu_f(g[4 * q + 3] * a.w) * (u[4 * q + 3] * b.w));
          }
      }
    }
  } else {
    const int cb = n0 + wn * WCOLS + cq;
    float4 sy[FN][4];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sy[j][q] = SC ? *(const float4*)(sc0 + cb + j * 32 + 8 * q) : make_float4(1.f, 1.f, 1.f, 1.f);
    float* Yb = ks == 0 ? (float*)out : out2 + (size_t)(ks - 1) * max_rows * N;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = lr + i * 32;
      if (row < rows) {
        float* Y = Yb + (size_t)(rbeg + row) * N + cb;
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& y = acc[i][j];
            const float4 c = sy[j][q];
            *(float4*)(Y + j * 32 + 8 * q) = make_float4(y[4 * q] * c.x, y[4 * q + 1] * c.y,
                                                         y[4 * q + 2] * c.z, y[4 * q + 3] * c.w);
          }
      }
    }
  }
}

// LDS buffers of one ring (or of the staged epilogue), by position.
struct Ring {
  u32x4 *b0, *b1, *b2, *b3, *b4, *b5;
};
__device__ __forceinline__ u32x4* ring(int h, const Ring& r) {
  return h == 0 ? r.b0 : h == 1 ? r.b1 : h == 2 ? r.b2 : h == 3 ? r.b3 : h == 4 ? r.b4 : r.b5;
}

// Staged tile epilogue (LDS-direct kernel).  The accumulator layout makes a
// direct store touch 32 rows per instruction, 8 or 16 bytes each; here the
// outputs pass through LDS so that consecutive threads store consecutive
// 16-B pieces of one output row and every store instruction covers whole
// 128-B lines.  Pass i takes the 32-row block i of every wave: each wave
// writes those rows' finished outputs (same arithmetic as store_tile) into
// the LDS region of its wave row, the block synchronises, and the 256
// threads store the rows (rows past the tile's end are skipped).  LDS row r
// keeps its 16-B chunk c at slot c ^ (r & 7).  With 2 WM regions the passes
// alternate between two sets and need one barrier each; with WM regions a
// second barrier ends every pass.  The regions are ring buffers: a first
// barrier makes sure no wave still reads the last stage.  Passes past the
// tile's last row (the same for every wave) are skipped.
template <int BM, int BN, int BNT, int WM, int WN, bool GLU>
struct StagedEpi {
  static constexpr int ES = GLU ? 2 : 4;                  // bf16 h or fp32 y
  static constexpr int OC = GLU ? BN : BNT;               // output columns per tile
  static constexpr int RB = OC * ES;                      // bytes per output row
  static constexpr int NC = RB / 16;                      // 16-B chunks per row
  static constexpr int PASS = 32 * RB;                    // bytes per region and pass
};

template <int BM, int BN, int BNT, int WM, int WN, int FM, int FN, bool GLU, bool SC, bool DB>
__device__ __forceinline__ void store_tile_staged(const f32x16 (&acc)[FM][FN],
                                                  void* __restrict__ out,
                                                  float* __restrict__ out2, int ks, int max_rows,
                                                  int N, int rbeg, int rows, int n0, int wm,
                                                  int wn, int lane, int tid,
                                                  const float* __restrict__ sc0,
                                                  const float* __restrict__ sc1,
                                                  const Ring& reg) {
  using E = StagedEpi<BM, BN, BNT, WM, WN, GLU>;
  constexpr int FNO = GLU ? FN / 2 : FN;                  // 32-column output blocks per wave
  constexpr int WOC = E::OC / WN;                         // output columns per wave
  constexpr int WROWS = BM / WM;
  static_assert(E::NC >= 8 && E::NC % 8 == 0 && WOC == 32 * FNO, "staged epilogue shape");
  const int r = lane & 31;
  const int cq = 4 * (lane >> 5);
  float4 sa[FNO][4], sb[FNO][4];
#pragma unroll
  for (int j = 0; j < FNO; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = n0 + wn * WOC + 32 * j + 8 * q + cq;
      sa[j][q] = SC ? *(const float4*)(sc0 + c) : make_float4(1.f, 1.f, 1.f, 1.f);
      sb[j][q] = (SC && GLU) ? *(const float4*)(sc1 + c) : make_float4(1.f, 1.f, 1.f, 1.f);
    }
  char* obase = GLU ? (char*)out
                    : (char*)(ks == 0 ? (float*)out : out2 + (size_t)(ks - 1) * max_rows * N);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (32 * i >= rows) break;   // no wave holds a live row in this or a later pass
    char* R = (char*)ring((DB ? (i & 1) * WM : 0) + wm, reg);
#pragma unroll
    for (int j = 0; j < FNO; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int byte = (wn * WOC + 32 * j + 8 * q + cq) * E::ES;
        char* p = R + r * E::RB + (((byte >> 4) ^ (r & 7)) << 4) + (byte & 15);
        const float4 a = sa[j][q], b = sb[j][q];
        if constexpr (GLU) {
          const f32x16& g = acc[i][j];
          const f32x16& u = acc[i][j + FNO];
          *(uint2*)p = make_uint2(bf16x2_bits(silu_f(g[4 * q] * a.x) * (u[4 * q] * b.x),
                                              silu_f(g[4 * q + 1] * a.y) * (u[4 * q + 1] * b.y)),
                                  bf16x2_bits(silu_f(g[4 * q + 2] * a.z) * (u[4 * q + 2] * b.z),
                                              silu_f(g[4 * q + 3] * a.w) * (u[4 * q + 3] * b.w)));
        } else {
          const f32x16& y = acc[i][j];
          *(float4*)p = make_float4(y[4 * q] * a.x, y[4 * q + 1] * a.y, y[4 * q + 2] * a.z,
                                    y[4 * q + 3] * a.w);
        }
      }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WM; ++w) {
      const char* R2 = (const char*)ring((DB ? (i & 1) * WM : 0) + w, reg);
#pragma unroll
      for (int e0 = 0; e0 < 32 * E::NC; e0 += kThreads) {
        const int e = e0 + tid;
        const int rr = e / E::NC, cc = e % E::NC;
        const int row = w * WROWS + 32 * i + rr;
        if (row < rows) {
          const u32x4 v = *(const u32x4*)(R2 + rr * E::RB + ((cc ^ (rr & 7)) << 4));
          u32x4* dst = (u32x4*)(obase + ((size_t)(rbeg + row) * N + n0) * E::ES + cc * 16);
          // fp32 y is read back only by the combine, after the whole
          // projection: non-temporal stores (DeepSeek-V3 down -3 %)
          if constexpr (GLU)
            *dst = v;
          else
            __builtin_nontemporal_store(v, dst);
        }
      }
    }
    if constexpr (!DB) {
      if (i + 1 < FM) __syncthreads();
    }
  }
}

// GLU = true : out = H [rows][N] (type T),  h = silu(A W1^T) * (A W3^T)
// GLU = false: out = Y [rows][N] (fp32),    y = A W2^T
// Work entry: {g | n_idx << 10, first row of the M-tile inside group g}.
template <typename T, int BM, int BN, int WM, int WN, bool GLU>
__global__ __launch_bounds__(kThreads) void k_moe_gemm(
    const T* __restrict__ A, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const int2* __restrict__ work,
    const int32_t* __restrict__ nwork, const T* __restrict__ B0, const T* __restrict__ B1,
    const T* __restrict__ B0_last, const T* __restrict__ B1_last, int g_last, int K, int N,
    int max_rows, int ksplit, int round, void* __restrict__ out, float* __restrict__ out2) {
  constexpr int NT = kThreads;
  constexpr int BNT = GLU ? 2 * BN : BN;
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-B chunk
  constexpr int BK = 8 * EPC;                  // elements per stage (128 B)
  constexpr int CA = BM * 8 / NT, CB = BNT * 8 / NT;   // 16-B chunks per thread per stage
  constexpr int WROWS = BM / WM, WCOLS = BNT / WN;
  constexpr int FM = WROWS / 32, FN = WCOLS / 32;
  constexpr int NF = FM + FN;                          // fragments per substep
  static_assert(WM * WN == 4, "four waves");
  static_assert(BM % 32 == 0 && BNT % 32 == 0 && BN % 32 == 0, "32-row load blocks");

  static_assert(FM >= 1 && FN >= 1 && (!GLU || FN % 2 == 0), "wave tile");
  static_assert(CA >= 1 && CB >= 1 && (BM * 8) % NT == 0 && (BNT * 8) % NT == 0, "tile loads");
  static_assert(!GLU || BN % (NT / 8) == 0, "gate/up halves split on thread rows");
  __shared__ u32x4 smem[2][(BM + BNT) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * WROWS;
  const int c16 = tid & 7;
  // this lane's fragment row bases (in 16-B chunks) and swizzled chunk per substep
  const int fa = (arow0 + (lane & 31)) * 8;
  const int fb = (BM + (GLU ? wn * (BN / WN) : wn * WCOLS) + (lane & 31)) * 8;
  int cs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) cs[q] = (2 * q + (lane >> 5)) ^ swz(lane & 31);
  // Blocks are dispatched round-robin over the 8 XCDs and run one per CU:
  // the i-th block of XCD x takes list entry (i / cx) * round + x * cx + i % cx
  // (cx = CUs per XCD, round = 8 cx), so in every round each XCD works on cx
  // consecutive entries of the list.
  const int cx = round >> 3;
  const int xi = blockIdx.x >> 3;
  const int t = (xi / cx) * round + (blockIdx.x & 7) * cx + (xi % cx);
  if (t >= nwork[0]) return;
  const int Kc = K / ksplit;                     // K range of one split (multiple of 2 BK)
  const int nk = Kc / BK;
  const size_t bstep = (size_t)(NT / 8) * K;   // element distance between a thread's B rows
  {
    const int2 wi = work[t];
    const int g = wi.x & 1023;
    const int n0 = ((wi.x >> 10) & 16383) * BN;
    // bf16: N-tile n starts its K loop at stage n mod nk, as in the LDS-direct
    // kernel (decode-shaped down projection, 4-KB weight rows: 1159 -> 1113 us)
    const int rot = sizeof(T) == 2 ? ((wi.x >> 10) & 16383) % nk : 0;
    const int ks = (int)((uint32_t)wi.x >> 24);   // K split of this entry
    const int kbeg = ks * Kc;
    const int gbeg = min(max(offsets[g], 0), max_rows);
    const int rbeg = gbeg + wi.y;
    const int gend = min(max(offsets[g + 1], gbeg), max_rows);
    const int rows = min(tile_height(gend - gbeg, BM), gend - rbeg);
    const T* w0 = ((g == g_last) ? B0_last : B0 + (size_t)g * N * K) + kbeg;
    const T* w1 = GLU ? ((g == g_last) ? B1_last : B1 + (size_t)g * N * K) + kbeg : nullptr;
    // per-thread source rows (64-bit addresses: an operand may hold 2^31
    // elements or more).  Rows past the tile's end re-read its first row:
    // their outputs are never stored, and each output row depends only on
    // its own A row.
    const T* oa[CA];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int r = (tid >> 3) + i * (NT / 8);
      int src = rbeg + (r < rows ? r : 0);
      if (row_token) src = row_token[src];
      oa[i] = A + (size_t)src * K + kbeg + c16 * EPC;
    }
    const T* pb0 = w0 + (size_t)(n0 + (tid >> 3)) * K + c16 * EPC;
    const T* pb1 = GLU ? w1 + (size_t)(n0 + (tid >> 3)) * K + c16 * EPC : nullptr;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // live 32-row blocks of this wave's part of the tile
    const int nv = min(FM, max(0, (rows - arow0 + 31) >> 5));
    auto* sm2 = reinterpret_cast<u32x4 (*)[1]>(&smem[0][0]);
#define MOE_MAIN_LOOP(NV_)                                                                   \
  main_loop<T, NV_, BM, BN, CA, CB, FM, FN, GLU>(acc, sm2, oa, pb0, pb1, bstep, nk, fa, fb, cs, \
                                                 tid, rot)
    if (nv >= FM) {
      MOE_MAIN_LOOP(FM);
    } else if (nv == 0) {
      MOE_MAIN_LOOP(0);
    } else {
      if constexpr (FM > 1) { if (nv == 1) MOE_MAIN_LOOP(1); }
      if constexpr (FM > 2) { if (nv == 2) MOE_MAIN_LOOP(2); }
      if constexpr (FM > 3) { if (nv == 3) MOE_MAIN_LOOP(3); }
    }
#undef MOE_MAIN_LOOP

    store_tile<T, BN, BNT, WN, FM, FN, GLU>(acc, out, out2, ks, max_rows, N, rbeg, rows, arow0,
                                            n0, wn, lane);
  }
}

// ------------------------------------------------------- LDS-DMA variant
// bf16 activations, bf16 or FP8 (E4M3) weights; tiles with BM, BNT multiples
// of 32.  A stage covers 64 K-elements (KB = 128) or 32 (KB = 64): KB bytes of
// every A row and, for bf16 weights, of every B row (KB / 2 bytes for FP8).
// The A parts of NBA stages and the B parts of NBB stages live in two rings
// of distinct LDS arrays, so the operand with the longer memory latency can
// be fetched further ahead than the other.  global_load_lds moves
// 16 B per lane from global memory straight into LDS (lane L of one wave
// instruction fills bytes [16 L, 16 L + 16) of a 1 KB block = 1024 / rowbytes
// rows), so stages never pass through registers.  LDS row r keeps chunk c
// (16 B) at slot c ^ swz(r); the lane that fills a slot fetches the matching
// chunk, and the fragment reads are bank-conflict free for 8- and 16-lane
// LDS service.  FP8 fragments (8 bytes per lane) are widened to bf16 in
// registers (exact: every E4M3 value is a bf16 value); the per-output-channel
// scales are applied to the fp32 accumulators in the epilogue.
//
// Iteration s (A part of stage s in A buffer s mod NBA, B part in B buffer
// s mod NBB):
//   wait until this wave's copies of stage s have landed (later copies may
//   still be in flight) and its LDS reads are done
//   barrier: every wave's copies of stage s are visible, and the buffers of
//   stage s - 1 are no longer read
//   start the copies of A part s + NBA - 1 and B part s + NBB - 1 into the
//   buffers stage s - 1 used
//   per k16 substep: MFMA the previous substep's fragments | read this one's
// Copies past the last stage re-fetch it (in bounds, never read), and the
// prologue issues stand-in copies in place of negative stages, so every
// wave always has the same number of copies in flight.
template <int RB>
__device__ __forceinline__ int swz_rb(int r) {       // RB = row bytes per stage
  if constexpr (RB == 64) return ((r >> 1) ^ (r >> 3)) & 3;
  else if constexpr (RB == 128) return swz(r);
  else return r & 15;                                // 256-B rows span all banks
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 left at its maximum, lgkmcnt 11:8 = 0).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// Geometry of one stage.  A rows hold KB bytes (bf16), B rows KB or KB / 2.
template <int BM, int BNT, int KB, bool Q8>
struct StageGeo {
  static constexpr int RBA = KB, RBB = Q8 ? KB / 2 : KB;        // row bytes
  static constexpr int CPA = RBA / 16, CPB = RBB / 16;          // 16-B chunks per row
  static constexpr int RPA = 64 / CPA, RPB = 64 / CPB;          // rows per copy instruction
  static constexpr int CA = BM / (4 * RPA), CB = BNT / (4 * RPB);   // copies per wave
  static constexpr int BOFF = BM * CPA;                          // first B slot
  static constexpr int SZ = BM * CPA + BNT * CPB;                // 16-B slots per stage
};

// Copies through buffer loads: a wave-uniform base (a buffer descriptor in
// SGPRs) plus a 32-bit per-lane byte offset that stays fixed for the whole
// K loop; the stage's K position is the descriptor's scalar offset.  The
// loop then spends no VALU work on addresses (the 64-bit per-lane form adds
// one 64-bit add per copy, and register pressure makes the compiler reuse
// one address register pair, so every copy waits for the previous one to
// read its address).  Valid when every offset of the operand stays below
// 2^32 bytes from its base; the launcher checks that on the host.
__device__ __forceinline__ void buf_lds16(const void* base, uint32_t off, uint32_t soff,
                                          void* lds) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xffffffff,
                                        0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, soff, 0, 0);
}
// Copy sources of a stage part: per copy a per-lane pointer (PtrSrc), or a
// wave-uniform base and a per-lane byte offset (BufSrc, bf16 operands).
template <typename T, int N>
struct PtrSrc {
  const T* p[N];
};
template <int N>
struct BufSrc {
  const void* base[N];
  uint32_t off[N];
};

// Copies of one stage's A or B part: instruction i of wave w fills A rows
// (w CA + i) RPA .. + RPA of an A buffer, or B rows (w CB + i) RPB .. + RPB
// of a B buffer.  pa[i], pb[i]: this lane's source of copy i at stage 0;
// koff is the stage's first K element.
template <int BM, int BNT, int KB, bool Q8, typename AL, int N>
__device__ __forceinline__ void dma_a(u32x4* buf, const PtrSrc<uint16_t, N>& pa, int koff,
                                      int wave, AL alive) {
  using G = StageGeo<BM, BNT, KB, Q8>;
  static_assert(N == G::CA, "A copies");
#pragma unroll
  for (int i = 0; i < G::CA; ++i)
    if ((uint32_t)alive & (1u << i))
      __builtin_amdgcn_global_load_lds((const void*)(pa.p[i] + koff),
                                       (void*)(buf + ((wave * G::CA + i) * G::RPA) * G::CPA), 16,
                                       0, 0);
}
template <int BM, int BNT, int KB, bool Q8, typename TB, int N>
__device__ __forceinline__ void dma_b(u32x4* buf, const PtrSrc<TB, N>& pb, int koff, int wave) {
  using G = StageGeo<BM, BNT, KB, Q8>;
  static_assert(N == G::CB, "B copies");
#pragma unroll
  for (int i = 0; i < G::CB; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(pb.p[i] + koff),
                                     (void*)(buf + ((wave * G::CB + i) * G::RPB) * G::CPB), 16,
                                     0, 0);
}

// Eight E4M3 bytes -> eight bf16 in MFMA operand order (byte i is element i),
// two per v_cvt_scalef32_pk_bf16_fp8 with scale 1 (exact: every E4M3 value
// is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ u32x4 widen_e4m3(uint2 v) {
  return u32x4{e4m3x2_bf16x2<false>(v.x), e4m3x2_bf16x2<true>(v.x), e4m3x2_bf16x2<false>(v.y),
               e4m3x2_bf16x2<true>(v.y)};
}

// Fragments of k16 substep q.  A (and bf16 B) reads are 16 B at slot cs; FP8
// B reads are 8 B: half (lane / 32) of chunk q at slot csb.
template <int NA, int FM, int FN, int BN, bool GLU, int CPA, int CPB, bool Q8>
__device__ __forceinline__ void load_frags_dma(u32x4* f, const u32x4* pa, const u32x4* pb,
                                               int cs, int csb, int half) {
  constexpr int FNH = GLU ? FN / 2 : FN;
#pragma unroll
  for (int i = 0; i < NA; ++i) f[i] = pa[i * 32 * CPA + cs];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int rr = GLU ? ((j < FNH) ? j * 32 : BN + (j - FNH) * 32) : j * 32;
    if constexpr (Q8) {
      const uint2 v = *((const uint2*)(pb + rr * CPB + csb) + half);
      f[FM + j] = widen_e4m3(v);
    } else {
      f[FM + j] = pb[rr * CPB + cs];
    }
  }
}


// Per-lane fragment addressing: A rows fa + 32 i, B rows fb + rr (both in
// slots of their region), swizzled chunk per substep.
struct FragAddr {
  int fa, fb, half;
  int rot;                  // first K stage of the tile's loop (stages taken cyclically)
  int cs[8], csb[8];
};

// MFMAs and fragment reads of one stage held in `cur`: per k16 substep, MFMA
// the previous substep's fragments while reading this one's.
template <int NV, int BM, int BN, int BNT, int FM, int FN, bool GLU, int KB, bool Q8>
__device__ __forceinline__ void stage_mma(f32x16 (&acc)[FM][FN], const u32x4* curA,
                                          const u32x4* curB, u32x4 (&f0)[FM + FN],
                                          u32x4 (&f1)[FM + FN], const FragAddr& fr,
                                          bool with_copies) {
  using G = StageGeo<BM, BNT, KB, Q8>;
  constexpr int NSUB = KB / 32;              // k16 substeps per stage
  const u32x4* pa = curA + fr.fa;
  const u32x4* pb = curB + fr.fb;
#pragma unroll
  for (int q = 0; q < NSUB; q += 2) {
    load_frags_dma<NV, FM, FN, BN, GLU, G::CPA, G::CPB, Q8>(f0, pa, pb, fr.cs[q], fr.csb[q],
                                                             fr.half);
    mma_substep<uint16_t, NV, FM, FN>(acc, f1);
    load_frags_dma<NV, FM, FN, BN, GLU, G::CPA, G::CPB, Q8>(f1, pa, pb, fr.cs[q + 1],
                                                             fr.csb[q + 1], fr.half);
    mma_substep<uint16_t, NV, FM, FN>(acc, f0);
  }
  constexpr int NM = NV * FN;
  constexpr int ND = NV + FN;
  constexpr int NG = G::CA + G::CB;
  if (with_copies) {
    if constexpr (NSUB == 2) {
      sched_substep<NM, ND, NG, 0>();
      sched_substep<NM, ND, 0, 0>();
    } else if constexpr (NSUB == 4) {
      sched_substep<NM, ND, NG / 2, 0>();
      sched_substep<NM, ND, NG - NG / 2, 0>();
      sched_substep<NM, ND, 0, 0>();
      sched_substep<NM, ND, 0, 0>();
    } else {                                 // 8 substeps: copies over the first four
      sched_substep<NM, ND, NG / 4, 0>();
      sched_substep<NM, ND, NG / 4, 0>();
      sched_substep<NM, ND, NG / 4, 0>();
      sched_substep<NM, ND, NG - 3 * (NG / 4), 0>();
#pragma unroll
      for (int q = 4; q < NSUB; ++q) sched_substep<NM, ND, 0, 0>();
    }
  } else {
#pragma unroll
    for (int q = 0; q < NSUB; ++q) sched_substep<NM, ND, 0, 0>();
  }
}

constexpr int gcd_i(int a, int b) { return b ? gcd_i(b, a % b) : a; }


// One iteration of the ring (see above) for stage s = s0 + h, h a
// compile-time position in the ring period.
template <int NV, int BM, int BN, int BNT, int FM, int FN, bool GLU, int KB, int NBA, int NBB,
          bool Q8, typename TB, int H, typename PA, typename PB, typename AL>
__device__ __forceinline__ void ring_step(f32x16 (&acc)[FM][FN], const Ring& ra, const Ring& rb,
                                          const PA& pa,
                                          const PB& pb,
                                          int s, int nk, u32x4 (&f0)[FM + FN],
                                          u32x4 (&f1)[FM + FN], const FragAddr& fr, int wave,
                                          AL alive) {
  using G = StageGeo<BM, BNT, KB, Q8>;
  constexpr int BK = KB / 2;                 // K-elements per stage
  // Each iteration copies the part of the shallower ring first (A on
  // equal depths).  The last copy stage s needs is that part of stage s,
  // followed by the other part's copies of the same iteration (unless the
  // depths are equal: then it is the B part, the iteration's last copy) and
  // by min(NBA, NBB) - 2 more iterations of copies.
  constexpr int NBS = NBA < NBB ? NBA : NBB;
  constexpr int WAITN = (NBA < NBB ? G::CB : NBA > NBB ? G::CA : 0) + (NBS - 2) * (G::CA + G::CB);
  wait_vm_lgkm<WAITN>();
  __builtin_amdgcn_s_barrier();
  const int ta = s + NBA - 1, tb = s + NBB - 1;
  if constexpr (NBA > NBB)
    dma_b<BM, BNT, KB, Q8, TB>(ring((H + NBB - 1) % NBB, rb), pb,
                               kstage(tb < nk ? tb : nk - 1, fr.rot, nk) * BK,
                               wave);
  dma_a<BM, BNT, KB, Q8>(ring((H + NBA - 1) % NBA, ra), pa,
                         kstage(ta < nk ? ta : nk - 1, fr.rot, nk) * BK, wave,
                         alive);
  if constexpr (NBA <= NBB)
    dma_b<BM, BNT, KB, Q8, TB>(ring((H + NBB - 1) % NBB, rb), pb,
                               kstage(tb < nk ? tb : nk - 1, fr.rot, nk) * BK,
                               wave);
  if constexpr (NV > 0)
    stage_mma<NV, BM, BN, BNT, FM, FN, GLU, KB, Q8>(acc, ring(H % NBA, ra), ring(H % NBB, rb),
                                                    f0, f1, fr, true);
}

template <int NV, int BM, int BN, int BNT, int FM, int FN, bool GLU, int KB, int NBA, int NBB,
          bool Q8, typename TB, typename PA, typename PB, typename AL, int... Hs>
__device__ __forceinline__ void ring_period(f32x16 (&acc)[FM][FN], const Ring& ra,
                                            const Ring& rb,
                                            const PA& pa,
                                            const PB& pb,
                                            int s0, int nk, int limit, u32x4 (&f0)[FM + FN],
                                            u32x4 (&f1)[FM + FN], const FragAddr& fr, int wave,
                                            AL alive, std::integer_sequence<int, Hs...>) {
  // limit: stages of this period to run (the whole period in the loop, the
  // remainder in the tail); uniform across the block
  ((Hs < limit ? ring_step<NV, BM, BN, BNT, FM, FN, GLU, KB, NBA, NBB, Q8, TB, Hs>(
                     acc, ra, rb, pa, pb, s0 + Hs, nk, f0, f1, fr, wave, alive)
               : (void)0),
   ...);
}

template <int NV, int BM, int BN, int BNT, int FM, int FN, bool GLU, int KB, int NBA, int NBB,
          bool Q8, typename TB, typename PA, typename PB, typename AL>
__device__ __forceinline__ void main_loop_dma(f32x16 (&acc)[FM][FN], const Ring& ra,
                                              const Ring& rb,
                                              const PA& pa,
                                              const PB& pb,
                                              int nk, const FragAddr& fr, int wave,
                                              AL alive) {
  static_assert(NBA >= 2 && NBB >= 2, "rings of at least two buffers");
  constexpr int NF = FM + FN;
  constexpr int BK = KB / 2;
  constexpr int P = NBA / gcd_i(NBA, NBB) * NBB;       // ring period
  // Prologue: virtual iterations i = -(max(NBA, NBB) - 1) .. -1 issue what
  // iteration i would (A part i + NBA - 1, B part i + NBB - 1); a negative
  // stage is a stand-in copy of stage 0 into the buffer it would use.
  constexpr int NBM = NBA > NBB ? NBA : NBB;
#pragma unroll
  for (int i = -(NBM - 1); i < 0; ++i) {
    const int sa = i + NBA - 1, sb = i + NBB - 1;
    if constexpr (NBA > NBB)
      dma_b<BM, BNT, KB, Q8, TB>(ring(((sb % NBB) + NBB) % NBB, rb), pb,
                                 kstage(sb < 0 ? 0 : (sb < nk ? sb : nk - 1), fr.rot, nk) * BK,
                                 wave);
    dma_a<BM, BNT, KB, Q8>(ring(((sa % NBA) + NBA) % NBA, ra), pa,
                           kstage(sa < 0 ? 0 : (sa < nk ? sa : nk - 1), fr.rot, nk) * BK, wave,
                           alive);
    if constexpr (NBA <= NBB)
      dma_b<BM, BNT, KB, Q8, TB>(ring(((sb % NBB) + NBB) % NBB, rb), pb,
                                 kstage(sb < 0 ? 0 : (sb < nk ? sb : nk - 1), fr.rot, nk) * BK,
                                 wave);
  }
  u32x4 f0[NF], f1[NF];
#pragma unroll
  for (int x = 0; x < NF; ++x) f1[x] = u32x4{0u, 0u, 0u, 0u};
  const int nfull = nk - nk % P;
  for (int s0 = 0; s0 < nfull; s0 += P)
    ring_period<NV, BM, BN, BNT, FM, FN, GLU, KB, NBA, NBB, Q8, TB>(
        acc, ra, rb, pa, pb, s0, nk, P, f0, f1, fr, wave, alive,
        std::make_integer_sequence<int, P>{});
  if (nfull < nk)
    ring_period<NV, BM, BN, BNT, FM, FN, GLU, KB, NBA, NBB, Q8, TB>(
        acc, ra, rb, pa, pb, nfull, nk, nk - nfull, f0, f1, fr, wave, alive,
        std::make_integer_sequence<int, P>{});
  if constexpr (NV > 0) mma_substep<uint16_t, NV, FM, FN>(acc, f1);
  wait_vm_lgkm<0>();   // no copy may still be landing when the block ends
}

// TB = uint16_t (bf16 weights) or uint8_t (E4M3 weights, Q8, with scales
// sc0/sc1 [G][N] and sc0l/sc1l [N] for group g_last).
// DENSE: one group of max_rows rows and no work list (the router logits).
template <int BM, int BN, int WM, int WN, bool GLU, int KB, int NBUF, bool Q8, int NBB,
          bool DENSE>
__global__ __launch_bounds__(kThreads) void k_moe_gemm_dma(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const int2* __restrict__ work,
    const int32_t* __restrict__ nwork, const void* __restrict__ B0v,
    const void* __restrict__ B1v, const void* __restrict__ B0lv,
    const void* __restrict__ B1lv, int g_last, int K, int N, int max_rows, int ksplit,
    int round, void* __restrict__ out, float* __restrict__ out2,
    const float* __restrict__ sc0, const float* __restrict__ sc1,
    const float* __restrict__ sc0l, const float* __restrict__ sc1l) {
  using T = uint16_t;
  using TB = typename std::conditional<Q8, uint8_t, uint16_t>::type;
  constexpr int BNT = GLU ? 2 * BN : BN;
  using G = StageGeo<BM, BNT, KB, Q8>;
  constexpr int WROWS = BM / WM, WCOLS = BNT / WN;
  constexpr int FM = WROWS / 32, FN = WCOLS / 32;
  static_assert(WM * WN == 4 && (KB == 64 || KB == 128 || (Q8 && KB == 256)) && (!Q8 || KB >= 128),
                "four waves; A rows of 64 or 128 B (256 B with FP8 weights, whose rows are half)");
  static_assert(NBUF >= 2 && NBUF <= 4 && NBB >= 2 && NBB <= 6,
                "A ring of 2..4 buffers, B ring of 2..6");
  static_assert(G::CA >= 1 && G::CB >= 1 && BM % (4 * G::RPA) == 0 && BNT % (4 * G::RPB) == 0 &&
                FM >= 1 && FN >= 1 && (!GLU || FN % 2 == 0), "tile shape");
  // GLU: a copy instruction's rows never straddle the W1 / W3 halves
  static_assert(!GLU || BN % G::RPB == 0, "gate/up halves split on copy rows");
  // Buffers the rings do not use are never referenced, so they take no LDS.
  constexpr int SZA = BM * G::CPA, SZB = BNT * G::CPB;
  __shared__ u32x4 LA0[SZA], LA1[SZA], LA2[SZA], LA3[SZA];
  __shared__ u32x4 LB0[SZB], LB1[SZB], LB2[SZB], LB3[SZB], LB4[SZB], LB5[SZB];
  const Ring ra{LA0, LA1, NBUF > 2 ? LA2 : LA0, NBUF > 3 ? LA3 : LA0, LA0, LA0};
  const Ring rb{LB0, LB1, NBB > 2 ? LB2 : LB0, NBB > 3 ? LB3 : LB0, NBB > 4 ? LB4 : LB0,
                NBB > 5 ? LB5 : LB0};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * WROWS;
  FragAddr fr;
  fr.fa = (arow0 + (lane & 31)) * G::CPA;
  fr.fb = ((GLU ? wn * (BN / WN) : wn * WCOLS) + (lane & 31)) * G::CPB;
  fr.half = lane >> 5;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    fr.cs[q] = ((2 * q + (lane >> 5)) % G::CPA) ^ swz_rb<G::RBA>(lane & 31);
    fr.csb[q] = (q % G::CPB) ^ swz_rb<G::RBB>(lane & 31);
  }
  const int cx = round >> 3;
  const int xi = blockIdx.x >> 3;
  const int t = (xi / cx) * round + (blockIdx.x & 7) * cx + (xi % cx);
  // A dense product (no list: one group of max_rows rows, the router
  // logits) takes entry t as M-tile t % mt of N-tile (t / mt) % NN and
  // K-split t / (mt NN).
  int2 wi;
  if constexpr (DENSE) {
    const int mt = (max_rows + BM - 1) / BM, nn = N / BN;
    if (t >= mt * nn * ksplit) return;
    const int kt = t / (mt * nn), r = t - kt * (mt * nn);
    wi = make_int2(((r / mt) << 10) | (kt << 24), (r % mt) * BM);
  } else {
    if (t >= nwork[0]) return;
    wi = work[t];
  }
  const int Kc = K / ksplit;
  const int nk = Kc / (KB / 2);
  const int g = wi.x & 1023;
  const int n0 = ((wi.x >> 10) & 16383) * BN;
  // bf16 weights: N-tile n starts its K loop at stage n mod nk and takes the
  // stages cyclically (the same sum in another order), so the tiles running
  // at once read different 128-B pieces of their weight rows.  With every
  // tile at the same K offset, rows a multiple of 4 KB apart crowded a few
  // HBM channels, depending on where the weights sit in physical memory:
  // the Switch-shaped gate/up took 239 or 202 us by allocation, 204 us
  // rotated; the DeepSeek-V3 down projection 1832 -> 1704 us.  FP8 codes
  // keep the plain order (rotated: DeepSeek-V3 down and FP8 decode down
  // 1-2 % slower, the Switch shape 3-5 % faster).
  fr.rot = (DENSE || Q8) ? 0 : ((wi.x >> 10) & 16383) % nk;
  const int ks = (int)((uint32_t)wi.x >> 24);
  const int kbeg = ks * Kc;
  const int gbeg = DENSE ? 0 : min(max(offsets[g], 0), max_rows);
  const int rbeg = gbeg + wi.y;
  const int gend = DENSE ? max_rows : min(max(offsets[g + 1], gbeg), max_rows);
  const int rows = min(DENSE ? BM : tile_height(gend - gbeg, BM), gend - rbeg);
  const TB* B0 = (const TB*)B0v;
  const TB* B1 = (const TB*)B1v;
  const TB* w0 = ((g == g_last) ? (const TB*)B0lv : B0 + (size_t)g * N * K) + kbeg;
  const TB* w1 = GLU ? ((g == g_last) ? (const TB*)B1lv : B1 + (size_t)g * N * K) + kbeg : nullptr;

  // This lane's source of each copy: row (w C + i) RP + lane / CP of the
  // tile, chunk (lane % CP) ^ swz(row).  Rows past the tile's end re-read its
  // first row: their outputs are never stored.
  PtrSrc<T, G::CA> pa;
#pragma unroll
  for (int i = 0; i < G::CA; ++i) {
    const int r = (wave * G::CA + i) * G::RPA + lane / G::CPA;
    int src = rbeg + (r < rows ? r : 0);
    if (row_token) src = row_token[src];
    pa.p[i] = A + (size_t)src * K + kbeg + (((lane % G::CPA) ^ swz_rb<G::RBA>(r & 31)) * 8);
  }
  // A copies whose rows all lie past the tile's end are not issued (their
  // LDS rows feed only outputs that are never stored).  The wait counts stay
  // right as long as no A copy is among the copies a wait leaves in flight:
  // two A buffers, issued before the B part of the same iteration.
  // 256-row tiles on a 2 x 2 wave grid serve experts with many rows, where
  // nearly every tile is full: there a ragged tile keeps all its copies, so
  // it runs in step with the neighbouring tiles on its XCD (skipping made
  // the few ragged tiles finish early and raised the Mixtral gate/up
  // fetches from 4.7 to 6.2 GB per launch).
  constexpr bool kSkipA = !(BM == 256 && WM == 2);
  static_assert(G::CA < 32, "one mask bit per A copy");
  constexpr uint32_t kAllA = (1u << G::CA) - 1;
  uint32_t alive = kAllA;
  if constexpr (kSkipA && NBUF == 2 && NBUF <= NBB) {
#pragma unroll
    for (int i = 0; i < G::CA; ++i)
      if ((wave * G::CA + i) * G::RPA >= rows) alive &= ~(1u << i);
  }
  alive = __builtin_amdgcn_readfirstlane(alive);
  constexpr int EPC_B = 16 / sizeof(TB);             // B elements per 16-B chunk
  PtrSrc<TB, G::CB> pb;
#pragma unroll
  for (int i = 0; i < G::CB; ++i) {
    const int r = (wave * G::CB + i) * G::RPB + lane / G::CPB;
    const int c = ((lane % G::CPB) ^ swz_rb<G::RBB>(r & 31)) * EPC_B;
    if constexpr (GLU)
      pb.p[i] = (r < BN ? w0 + (size_t)(n0 + r) * K : w1 + (size_t)(n0 + r - BN) * K) + c;
    else
      pb.p[i] = w0 + (size_t)(n0 + r) * K + c;
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // 32-row blocks holding real rows; tiles 8 blocks tall run an even
  // count (one block past the rows at most: computed, never stored), which
  // halves the loop instantiations
  int nv = min(FM, max(0, (rows - arow0 + 31) >> 5));
  if constexpr (FM > 4) nv = min(FM, (nv + 1) & ~1);
  static_assert(FM <= 8, "at most eight 32-row blocks per wave");
#define MOE_DMA_LOOP(NV_, AL_)                                                                \
  main_loop_dma<NV_, BM, BN, BNT, FM, FN, GLU, KB, NBUF, NBB, Q8, TB>(acc, ra, rb, pa, pb, nk, fr, \
                                                                     wave, AL_)
#define MOE_DMA_NV(AL_)                                                                       \
  if (nv >= FM) {                                                                             \
    MOE_DMA_LOOP(FM, AL_);                                                                    \
  } else if (nv == 0) {                                                                       \
    MOE_DMA_LOOP(0, AL_);                                                                     \
  } else if constexpr (FM <= 4) {                                                             \
    if constexpr (FM > 1) { if (nv == 1) MOE_DMA_LOOP(1, AL_); }                              \
    if constexpr (FM > 2) { if (nv == 2) MOE_DMA_LOOP(2, AL_); }                              \
    if constexpr (FM > 3) { if (nv == 3) MOE_DMA_LOOP(3, AL_); }                              \
  } else {                                                                                    \
    if (nv == 2) MOE_DMA_LOOP(2, AL_);                                                        \
    if constexpr (FM > 4) { if (nv == 4) MOE_DMA_LOOP(4, AL_); }                              \
    if constexpr (FM > 6) { if (nv == 6) MOE_DMA_LOOP(6, AL_); }                              \
  }
  // With the mask a compile-time constant every copy is issued and the
  // copies stay interleaved with the MFMAs (no branches).
  const std::integral_constant<uint32_t, kAllA> all_a{};
  if constexpr (!kSkipA) {
    MOE_DMA_NV(all_a);
  } else if (rows >= BM) {
    MOE_DMA_LOOP(FM, all_a);
  } else {
    MOE_DMA_NV(alive);
  }
#undef MOE_DMA_NV
#undef MOE_DMA_LOOP
  const float* s0p = nullptr;
  const float* s1p = nullptr;
  if constexpr (Q8) {
    s0p = (g == g_last) ? sc0l : sc0 + (size_t)g * N;
    s1p = GLU ? ((g == g_last) ? sc1l : sc1 + (size_t)g * N) : nullptr;
  }
  // The down projection's fp32 rows go through the staged epilogue (ring
  // buffers that hold a whole pass); the gate/up tile's bf16 h is stored
  // directly, which measured as fast.
  using E = StagedEpi<BM, BN, BNT, WM, WN, GLU>;
  constexpr bool FA = SZA * 16 >= E::PASS, FB = SZB * 16 >= E::PASS;
  constexpr int NR = (FA ? 2 : 0) + (FB ? 2 : 0);
  if constexpr (!GLU && NR >= WM) {
    const Ring reg{FA ? LA0 : LB0, FA ? LA1 : LB1, FA && FB ? LB0 : LA0, FA && FB ? LB1 : LA1,
                   LA0, LA0};
    store_tile_staged<BM, BN, BNT, WM, WN, FM, FN, GLU, Q8, (NR >= 2 * WM)>(
        acc, out, out2, ks, max_rows, N, rbeg, rows, n0, wm, wn, lane, tid, s0p, s1p, reg);
  } else {
    store_tile<T, BN, BNT, WN, FM, FN, GLU, Q8>(acc, out, out2, ks, max_rows, N, rbeg, rows,
                                                arow0, n0, wn, lane, s0p, s1p);
  }
}

// ------------------------------------------------------- ping-pong variant
// Both projections of the large tiles (experts with hundreds of rows, bf16
// or E4M3 weights): 256 rows x 256 B rows per block (256 output columns of the down
// projection, or 128 gate and the 128 matching up columns), eight waves in
// two groups of four (one wave of each group per SIMD).  Group 0 owns rows
// [0, h) and group 1 rows [h, 2 h) of the tile, h = 16 ceil(rows / 32) (128
// on a full tile); wave wi owns 64 of the B rows: up to 8 x 4 accumulator
// blocks of 16x16 (128 registers), so two waves share a SIMD.  The products run on
// v_mfma_f32_16x16x32_bf16: under the power limit that sets the clock of a
// fully loaded GPU it sustains 6-10 % more than the 32x32x16 form at the
// same LDS bytes per product (it moves fewer accumulator bytes per flop).
//
// The two groups alternate between a memory phase (read the next 32 K of
// fragments from LDS into registers, issue global->LDS copies, wait) and a
// compute phase (32 MFMAs from registers only), offset by one phase and
// separated by block barriers: while one wave of a SIMD feeds the matrix
// core the other does its loads, so the matrix core never waits on an LDS
// read.
//
// Copies move whole 128-B lines (a stage is 64 K-elements: the address unit
// spends the same time on a half line as on a full one).  The A and B parts
// of a stage live in separate rings of 32 KB buffers, 2 for A and 3 for B
// (160 KB): A(S + 1) is issued in the first memory phase of stage S, B(S + 2)
// in the second, so the address unit sees an even load and the weight rows
// get two stages of lead.  Every wave copies 32 A rows and 32 B rows of each
// stage.  Its 128 x 64 wave tile reads 1.5 times the LDS bytes per MFMA of
// the 4-wave kernel's 128 x 128; the alternation hides the copies better
// than the 4-wave kernel's single wave per SIMD can (Mixtral-shaped gate/up
// 7 % faster, grouped and dense alike).
struct PPRing {
  static constexpr int BM = 256, BN = 256;    // token rows, output columns per tile
  static constexpr int NA = 2, NB = 3;        // ring depths (64-K stages)
  static constexpr int HS = 256 * 8;          // 16-B slots per 32 KB buffer
};

// Epilogue of a ping-pong wave tile (16x16 accumulator blocks, see k_moe_pp):
// acc[i][j][r] is the output of token row arow0 + 16 i + (lane & 15) and
// column cb + 16 j + r with cb the wave's first column + 4 (lane >> 4), so
// every lane stores runs of four consecutive outputs of one row and the 16
// lanes of one row offset together write 64 contiguous bytes of fp32 y (32
// of bf16 h).  Rows at or past `rows` (one past the last row this group
// owns) are masked per lane.
//   GLU : gate blocks j = 0, 1 and the matching up blocks j + 2; h =
//         silu(gate) * up, rounded once to bf16
//   else: y in fp32
// With SC (FP8 weights) the accumulators are first multiplied by the
// per-output-channel scales: gate by sc0[n], up by sc1[n], down by sc0[n].
template <bool GLU, bool SC>
__device__ __forceinline__ void store_tile_pp(const f32x4 (&acc)[8][4], void* __restrict__ out,
                                              int N, int rbeg, int rows, int arow0, int wcol0,
                                              int lane, const float* __restrict__ sc0,
                                              const float* __restrict__ sc1) {
  const int lr = arow0 + (lane & 15);
  const int cb = wcol0 + 4 * (lane >> 4);
  constexpr int NJ = GLU ? 2 : 4;
  float4 s0[NJ], s1[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    s0[j] = SC ? *(const float4*)(sc0 + cb + 16 * j) : make_float4(1.f, 1.f, 1.f, 1.f);
    s1[j] = (SC && GLU) ? *(const float4*)(sc1 + cb + 16 * j) : make_float4(1.f, 1.f, 1.f, 1.f);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = lr + 16 * i;
    if (row < rows) {
      if constexpr (GLU) {
        uint16_t* H = (uint16_t*)out + (size_t)(rbeg + row) * N + cb;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4& g = acc[i][j];
          const f32x4& u = acc[i][j + 2];
          const float4 a = s0[j], b = s1[j];
          store4_h<uint16_t>(H + 16 * j, silu_f(g[0] * a.x) * (u[0] * b.x),
                             silu_f(g[1] * a.y) * (u[1] * b.y), silu_f(g[2] * a.z) * (u[2] * b.z),
                             silu_f(g[3] * a.w) * (u[3] * b.w));
        }
      } else {
        float* Y = (float*)out + (size_t)(rbeg + row) * N + cb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4& y = acc[i][j];
          const float4 c = s0[j];
          *(float4*)(Y + 16 * j) = make_float4(y[0] * c.x, y[1] * c.y, y[2] * c.z, y[3] * c.w);
        }
      }
    }
  }
}

// LDS swizzle of the ping-pong kernel's 128-B rows: chunk c of row r at slot
// c ^ ((r >> 1) & 7).  Its 16x16x32 fragment reads put 16 lanes on 16
// consecutive rows at one chunk and four chunks in one instruction; with
// swz() that pattern measured 128 B/clk per CU on gfx950 (two-way bank
// conflicts), with this form 256 B/clk, the rate of contiguous reads.  Rows
// 2m and 2m + 1 share a slot and sit in opposite 128-B halves of a 256-B
// bank line.
__device__ __forceinline__ int swz_pp(int r) { return (r >> 1) & 7; }

// A barrier that no instruction is scheduled across (the compiler may
// otherwise hoist it past the MFMAs of a compute phase).
__device__ __forceinline__ void fenced_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// GLU = false: out = Y (fp32), y = A W2^T, N = d; tiles of 256 output
//              columns.  The entries of a tile split along K write their
//              parts to slots of out2, and k_tail_sum adds them up.
// GLU = true:  out = H (bf16), h = silu(A W1^T) * (A W3^T), N = F; tiles of
//              128 columns, the B tile holding their 128 W1 rows then their
//              128 W3 rows; wave wi owns gate columns 32 wi .. 32 wi + 31 and
//              the matching up columns, so SwiGLU runs on its accumulators.
// BUF: copies in buffer form (byte offsets below 2^32, checked by the launcher).
// Q8: the weights are E4M3 codes (64-B rows per stage, 16 rows per copy
// instruction), widened to bf16 in registers; the per-output-channel scales
// sc0 (W1 or W2) and sc1 (W3) multiply the accumulators in the epilogue.
template <bool GLU, bool BUF, bool Q8>
__global__ __launch_bounds__(512) void k_moe_pp(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const int2* __restrict__ work,
    const int32_t* __restrict__ nwork, const void* __restrict__ B0v,
    const void* __restrict__ B1v, const void* __restrict__ B0lv,
    const void* __restrict__ B1lv, int g_last, int K, int N, int max_rows,
    int round, void* __restrict__ out, float* __restrict__ out2,
    const float* __restrict__ sc0, const float* __restrict__ sc1,
    const float* __restrict__ sc0l, const float* __restrict__ sc1l) {
  using R = PPRing;
  using TB = typename std::conditional<Q8, uint8_t, uint16_t>::type;
  constexpr int CPB = Q8 ? 4 : 8;        // 16-B chunks per B row and stage
  constexpr int RPB = 64 / CPB;          // B rows per copy instruction
  constexpr int NCB = 32 / RPB;          // B copies per wave and stage
  constexpr int HSB = R::BM * CPB;       // 16-B slots per B buffer
  __shared__ u32x4 la[R::NA * R::HS];
  __shared__ u32x4 lb[R::NB * HSB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gp = wave >> 2, wi = wave & 3;
  // Blocks are dispatched round-robin over the 8 XCDs: in every round of
  // `round` blocks each XCD takes a contiguous run of the list.
  const int cx = round >> 3;
  const int xi = blockIdx.x >> 3;
  const int t = (xi / cx) * round + (blockIdx.x & 7) * cx + (xi % cx);
  if (t >= nwork[0]) return;
  const int2 wk = work[t];
  const int g = wk.x & 1023;
  constexpr int TBN = GLU ? R::BN / 2 : R::BN;   // output columns per tile
  const int n0 = ((wk.x >> 10) & 16383) * TBN;
  const int ks = (wk.x >> 24) & 15;           // part ks of 2^lg along K
  const int lg = (wk.x >> 28) & 7;
  const int Kc = K >> lg;
  const int kbeg = ks * Kc;
  const int nk = Kc / 64;
  const int gbeg = min(max(offsets[g], 0), max_rows);
  const int rbeg = gbeg + wk.y;
  const int gend = min(max(offsets[g + 1], gbeg), max_rows);
  const int rows = min(tile_height(gend - gbeg, R::BM), gend - rbeg);
  const TB* B0 = (const TB*)B0v;
  const TB* B1 = (const TB*)B1v;
  const TB* w0 = ((g == g_last) ? (const TB*)B0lv : B0 + (size_t)g * N * K) + kbeg;
  const TB* w1 = GLU ? ((g == g_last) ? (const TB*)B1lv : B1 + (size_t)g * N * K) + kbeg : w0;

  // This wave's copies: A rows wave * 32 + 8 i + lane / 8, chunk (lane % 8)
  // ^ swz_pp(row) of each 128-B row; B rows wave * 32 + RPB i + lane / CPB,
  // chunk (lane % CPB) ^ swz_pp(row) (bf16) or ^ swz_rb<64>(row) (FP8 codes)
  // (a copy's B rows lie in one of the W1 / W3 halves).  A rows past the tile's end re-read its first row
  // (their outputs are never stored).
  // element offsets of this lane's copies from A + kbeg and from w0 / w1
  size_t ea[4], eb[NCB];
  int dsa[4], dsb[NCB];
  bool bhi[NCB];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wave * 32 + i * 8 + lane / 8;
    const int c = ((lane % 8) ^ swz_pp(r)) * 8;
    int src = rbeg + (r < rows ? r : 0);
    if (GLU && row_token) src = row_token[src];
    ea[i] = (size_t)src * K + c;
    dsa[i] = (wave * 32 + i * 8) * 8;
  }
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const int r = wave * 32 + i * RPB + lane / CPB;
    const int c = ((lane % CPB) ^ (Q8 ? swz_rb<64>(r & 31) : swz_pp(r))) * (16 / (int)sizeof(TB));
    bhi[i] = GLU && wave * 32 + i * RPB >= TBN;
    eb[i] = (size_t)(n0 + (bhi[i] ? r - TBN : r)) * K + c;
    dsb[i] = (wave * 32 + i * RPB) * CPB;
  }
  const uint16_t* abase = A + kbeg;
  std::conditional_t<BUF, BufSrc<4>, PtrSrc<uint16_t, 4>> sa;
  std::conditional_t<BUF, BufSrc<NCB>, PtrSrc<TB, NCB>> sb;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BUF) {
      sa.base[i] = abase;
      sa.off[i] = (uint32_t)(ea[i] * 2);
    } else {
      sa.p[i] = abase + ea[i];
    }
  }
#pragma unroll
  for (int i = 0; i < NCB; ++i) {
    const TB* wb = bhi[i] ? w1 : w0;
    if constexpr (BUF) {
      sb.base[i] = wb;
      sb.off[i] = (uint32_t)(eb[i] * sizeof(TB));
    } else {
      sb.p[i] = wb + eb[i];
    }
  }
  // stage S: K elements [64 S, 64 S + 64) of the split (64 elements of
  // each row: 128 B of A, 64 sizeof(TB) B of W)
  auto copy_a = [&](int S) {
    u32x4* buf = la + (S % R::NA) * R::HS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (BUF)
        buf_lds16(sa.base[i], sa.off[i], (uint32_t)S * 128u, (void*)(buf + dsa[i]));
      else
        __builtin_amdgcn_global_load_lds((const void*)(sa.p[i] + S * 64),
                                         (void*)(buf + dsa[i]), 16, 0, 0);
    }
  };
  auto copy_b = [&](int S) {
    u32x4* buf = lb + (S % R::NB) * HSB;
#pragma unroll
    for (int i = 0; i < NCB; ++i) {
      if constexpr (BUF)
        buf_lds16(sb.base[i], sb.off[i], (uint32_t)S * (64u * (uint32_t)sizeof(TB)),
                  (void*)(buf + dsb[i]));
      else
        __builtin_amdgcn_global_load_lds((const void*)(sb.p[i] + S * 64),
                                         (void*)(buf + dsb[i]), 16, 0, 0);
    }
  };
  // 16x16x32 fragments: lane l holds 8 K-contiguous values of row l % 16 of
  // a 16-row block, K offset 8 (l / 16) inside the k32 substep (chunk
  // 4 hh + l / 16 of the 64-K stage for substep hh, swizzled).  A blocks i:
  // rows 128 gp + 16 i; B blocks j: rows 64 wi + 16 j (GLU: j = 0, 1 gate
  // rows 32 wi + 16 j, j = 2, 3 the matching up rows TBN + 32 wi + 16 (j -
  // 2)).  Every block starts at a multiple of 16: the bf16 swizzle of a
  // lane's rows depends on lane % 16 only, the FP8 one also on the block's
  // parity.
  // The tile's rows are split evenly between the groups in 16-row blocks:
  // group 0 takes rows [0, hrow), group 1 rows [hrow, rows), hrow = 16
  // ceil(rows / 32) (128 on a full tile).  On a partial tile both compute
  // phases then stay about equally long, so neither waits on the other's
  // memory phase more than the tile's rows require.
  const int hrow = min(128, ((rows + 31) >> 5) << 4);
  const int g0 = gp * hrow;                    // this group's first row
  const int ghi = min(rows, g0 + hrow);        // one past its last row
  const int ra = g0 + (lane & 15);
  int rb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    rb[j] = (GLU ? (j < 2 ? 32 * wi + 16 * j : TBN + 32 * wi + 16 * (j - 2)) : 64 * wi + 16 * j) +
            (lane & 15);
  int csw[2], csb[2][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    csw[hh] = (4 * hh + (lane >> 4)) ^ swz_pp(lane & 15);
    // FP8 rows (64 B): chunk 2 hh + l / 32 holds 16 codes, half (l / 16) % 2 the lane's 8
#pragma unroll
    for (int p = 0; p < 2; ++p)
      csb[hh][p] = (2 * hh + (lane >> 5)) ^ swz_rb<64>(16 * p + (lane & 15));
  }
  const int half = (lane >> 4) & 1;
  // live 16-row blocks of this group's rows: the rest skip their MFMAs
  const int nv = __builtin_amdgcn_readfirstlane(max(0, ghi - g0 + 15) >> 4);

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;
  u32x4 fa[8], fb[4];

  // prologue: A stage 0, B stages 0 and 1 landed in every wave; then group
  // 1 falls one phase behind group 0
  copy_a(0);
  copy_b(0);
  if (nk > 1) copy_b(1);
  wait_vm_lgkm<0>();
  fenced_barrier();
  if (gp == 1) fenced_barrier();
  // The K loop for a wave with NV live 16-row blocks (compile time, so a
  // full tile's compute phases are straight runs of MFMAs); every wave runs
  // the same copies and barriers whatever its NV.
  auto kloop = [&](auto nv_c) {
    constexpr int NV = decltype(nv_c)::value;
    for (int S = 0; S < nk; ++S) {
      const u32x4* ba = la + (S % R::NA) * R::HS;
      const u32x4* bb = lb + (S % R::NB) * HSB;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // ---- memory phase: fragments of k32 substep hh (live A blocks only)
#pragma unroll
        for (int i = 0; i < NV; ++i) fa[i] = ba[(ra + 16 * i) * 8 + csw[hh]];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (Q8)
            fb[j] = widen_e4m3(*((const uint2*)(bb + rb[j] * CPB + csb[hh][j & 1]) + half));
          else
            fb[j] = bb[rb[j] * 8 + csw[hh]];
        }
        // A(S + 1) goes into the A buffer stage S - 1 used, B(S + 2) into
        // the B buffer of stage S - 1: both were last read in the previous
        // phase of the other group, before the barrier that ended it.
        if (hh == 0) {
          if (S + 1 < nk) copy_a(S + 1);
          wait_vm_lgkm<NCB + 4>();              // LDS reads done; copies fly on
        } else if (S + 2 < nk) {
          copy_b(S + 2);
          wait_vm_lgkm<NCB>();                  // all but B(S + 2): stage S + 1 landed
        } else {
          wait_vm_lgkm<0>();
        }
        fenced_barrier();
        // ---- compute phase
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, fb[j]), __builtin_bit_cast(bf16x8, fa[i]), acc[i][j], 0,
                0, 0);
        __builtin_amdgcn_s_setprio(0);
        fenced_barrier();
      }
    }
  };
  switch (nv) {
    case 8: kloop(std::integral_constant<int, 8>{}); break;
    case 7: kloop(std::integral_constant<int, 7>{}); break;
    case 6: kloop(std::integral_constant<int, 6>{}); break;
    case 5: kloop(std::integral_constant<int, 5>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }
  if (gp == 0) fenced_barrier();              // both groups end on the same barrier count
  const float* s0p = nullptr;
  const float* s1p = nullptr;
  if constexpr (Q8) {
    s0p = (g == g_last) ? sc0l : sc0 + (size_t)g * N;
    s1p = GLU ? ((g == g_last) ? sc1l : sc1 + (size_t)g * N) : nullptr;
  }
  if constexpr (GLU) {
    store_tile_pp<true, Q8>(acc, out, N, rbeg, ghi, g0, n0 + 32 * wi, lane, s0p, s1p);
  } else if (lg == 0) {
    store_tile_pp<false, Q8>(acc, out, N, rbeg, ghi, g0, n0 + 64 * wi, lane, s0p, nullptr);
  } else {
    // A tile split along K (the work list's last tiles): part ks goes to
    // slot (ti 2^lg + ks) of `out2` (slots of BM x BN floats, row-major);
    // k_tail_sum adds the parts in part order once every part has ended.
    const int ti = (t - nwork[1]) >> lg;       // split tile index
    store_tile_pp<false, Q8>(acc, out2 + (size_t)((ti << lg) + ks) * (R::BM * R::BN), R::BN, 0,
                             ghi, g0, 64 * wi, lane, Q8 ? s0p + n0 : nullptr, nullptr);
  }
}

// Sums the K parts of the split tiles into the output rows, in part order
// (a separate launch: the stream orders it after every part, with no
// device-scope fence inside the GEMM; such fences write back and invalidate
// an XCD's whole L2, and in the GEMM they cost more than the split saved).
// Block b takes rows [32 (b % 8), +32) of split tile b / 8: the grid is
// round / 2 x 8 blocks, as at most round / 2 tiles are split.
__global__ __launch_bounds__(256) void k_tail_sum(const int2* __restrict__ work,
                                                  const int32_t* __restrict__ nwork,
                                                  const int32_t* __restrict__ offsets,
                                                  int max_rows, int N,
                                                  const float* __restrict__ slots,
                                                  float* __restrict__ Y) {
  constexpr int BM = PPRing::BM, BN = PPRing::BN;
  const int total = nwork[0], base = nwork[1];
  if (total <= base) return;
  const int lg = (work[base].x >> 28) & 7;
  const int ti = blockIdx.x >> 3, band = blockIdx.x & 7;
  if (ti >= (total - base) >> lg) return;
  const int2 wk = work[base + (ti << lg)];
  const int g = wk.x & 1023;
  const int n0 = ((wk.x >> 10) & 16383) * BN;
  const int gbeg = min(max(offsets[g], 0), max_rows);
  const int rbeg = gbeg + wk.y;
  const int gend = min(max(offsets[g + 1], gbeg), max_rows);
  const int rows = min(tile_height(gend - gbeg, BM), gend - rbeg);
  const float* p = slots + (size_t)(ti << lg) * (BM * BN);
  for (int x = threadIdx.x; x < 32 * (BN / 4); x += 256) {
    const int r = band * 32 + x / (BN / 4), c = 4 * (x % (BN / 4));
    if (r >= rows) break;
    float4 a = *(const float4*)(p + r * BN + c);
    for (int k = 1; k < (1 << lg); ++k) {
      const float4 b = *(const float4*)(p + (size_t)k * (BM * BN) + r * BN + c);
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    *(float4*)(Y + (size_t)(rbeg + r) * N + n0 + c) = a;
  }
}

// Work list: for each group g, mt_g = ceil(rows_g / BM) M-tiles (of
// tile_height(rows_g, BM) rows, the last one taking the rest) times NN
// N-tiles, ordered by group, then M-groups of at most kMGroup M-tiles, then runs of NG neighbouring N-tiles,
// then N-tile, with the M-tiles of the group fastest.  The blocks of one
// XCD take a contiguous run of the list, so they hold a few N-tiles of all
// the M-tiles of an expert (up to kMGroup): with an expert of five M-tiles
// that keeps each weight slice and each activation tile in the XCD's L2
// while all its users run (N-tiles fastest had split the M-tiles of one
// N-tile across XCDs: 4.3 against 3.0 GB fetched per Mixtral-shaped
// gate/up launch).  One launch builds the lists of both projections.
//
// Group g's rows are [a_g, b_g) with the caller's offsets clamped to
// [0, max_rows] and made non-decreasing by a running maximum (b_g = the
// largest clamped end up to g, a_g = b_{g-1}), so the groups never overlap
// and the list never holds more than ceil(max_rows / BM) + G M-tiles per
// N-tile, whatever the offsets hold.  Block (0, 0) stores these bounds in
// `clean` [G+1]; the GEMMs read their rows from there.
struct WorkListArgs {
  int BM, NN, NG;
  int tail;           // largest K-split of the last tiles (a power of two; 1: none)
  int round;          // blocks per dispatch round
  int2* work;
  int32_t* nwork;     // [0] entries, [1] first split entry
};

// blockIdx.y picks the list; the kWorkSlices blocks of a list each rebuild
// the group scan (cheap, G <= 1024) and write every kWorkSlices-th run of
// 1024 entries.
constexpr int kWorkSlices = 8;
constexpr int kMGroup = 8;
__global__ __launch_bounds__(1024) void k_work_list(const int32_t* __restrict__ offsets, int G,
                                                    int max_rows, WorkListArgs l0,
                                                    WorkListArgs l1,
                                                    int32_t* __restrict__ clean) {
  const WorkListArgs& l = blockIdx.y == 0 ? l0 : l1;
  const int BM = l.BM, NN = l.NN, NG = l.NG;
  int2* __restrict__ work = l.work;
  int32_t* __restrict__ nwork = l.nwork;
  __shared__ int32_t sc[1024];
  __shared__ int32_t mts[1024];
  __shared__ int32_t bend[1024];
  __shared__ int32_t wsum[16];
  __shared__ int32_t hts[1024];
  const int g = threadIdx.x;
  const int lane = g & 63, wv = g >> 6;
  // running maximum of the clamped group ends (inclusive max-scan)
  const int a0 = min(max(offsets[0], 0), max_rows);
  int be = a0;
  if (g < G) be = max(a0, min(max(offsets[g + 1], 0), max_rows));
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(be, o);
    if (lane >= o) be = max(be, y);
  }
  if (lane == 63) wsum[wv] = be;
  __syncthreads();
  for (int i = 0; i < wv; ++i) be = max(be, wsum[i]);
  bend[g] = be;
  __syncthreads();
  int mt = 0;
  if (g < G) {
    const int a = g == 0 ? a0 : bend[g - 1];
    mt = MOE_CEIL_DIV(be - a, BM);
    hts[g] = tile_height(be - a, BM);
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      clean[g] = a;
      if (g == G - 1) clean[G] = be;
    }
  }
  mts[g] = mt;
  __syncthreads();                       // wsum is reused below
  // inclusive scan of the entry counts: in each wave by shuffles, then over
  // the 16 wave totals
  int v = mt * NN;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum[wv] = v;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wv; ++i) before += wsum[i];
  sc[g] = v + before;
  __syncthreads();
  const int total = sc[1023];
  const int nfull = NN / NG;
  // The q tiles after the last full dispatch round are split along K into
  // 2^lg parts (the largest power of two up to `tail` with q 2^lg <= round),
  // so that round ends after 1 / 2^lg of a tile instead of a whole one.
  int q = 0, lg = 0;
  if (l.tail > 1) {
    q = total % l.round;
    while ((2 << lg) <= l.tail && q * (2 << lg) <= l.round) ++lg;
    if (lg == 0) q = 0;
  }
  const int base = total - q;
  for (int e = blockIdx.x * 1024 + g; e < total; e += kWorkSlices * 1024) {
    int lo = 0, hi = G - 1;                     // first group with inclusive sum > e
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (sc[mid] > e) hi = mid; else lo = mid + 1;
    }
    const int gg = lo;
    const int m = mts[gg];
    const int j = e - (sc[gg] - m * NN);
    int mi, ni;
    // M-groups of at most kMGroup M-tiles; in a group, runs of NG N-tiles;
    // in a run, N-tile by N-tile with the group's M-tiles fastest
    const int g0 = (j / (kMGroup * NN)) * kMGroup;
    const int ms = min(kMGroup, m - g0);
    const int jj = j - g0 * NN;
    if (jj < ms * NG * nfull) {
      const int run = jj / (ms * NG), r = jj - run * ms * NG;
      ni = run * NG + r / ms;
      mi = g0 + r % ms;
    } else {                                    // the final, shorter run
      const int r = jj - ms * NG * nfull;
      ni = nfull * NG + r / ms;
      mi = g0 + r % ms;
    }
    const int x = gg | (ni << 10);
    if (e < base) {
      work[e] = make_int2(x, mi * hts[gg]);
    } else {                                    // split tile: its parts are adjacent
      for (int k = 0; k < (1 << lg); ++k)
        work[base + ((e - base) << lg) + k] = make_int2(x | (k << 24) | (lg << 28), mi * hts[gg]);
    }
  }
  if (blockIdx.x == 0 && g == 0) {
    nwork[0] = base + (q << lg);
    nwork[1] = base;
  }
}

// ------------------------------------------------------------------ launch
#ifndef MOE_CFG0_BM
#define MOE_CFG0_BM 256
#endif
// Depth of the weight-row ring of the 256-row tiles (two activation buffers).
#ifndef MOE_CFG0_NBB
#define MOE_CFG0_NBB 2
#endif
struct GemmPlan {
  int BM;
  int cfg;   // 0 = large, 1 = medium, 2 = small (decode), 3 = fp32
};

// Medium shapes (a few hundred rows per expert or fewer, HBM-bound) take
// 256-row tiles with the four waves side by side (1 x 4), so an expert's
// weight slice is streamed once even when it holds more than 128 rows, and
// 32-row blocks past the expert's rows cost no MFMA time on any wave.  bf16
// and FP8 weights share the plan (FP8 on 128-row 2 x 2 tiles, whose experts
// above 128 rows stream their weights twice, was 14 % slower on the
// DeepSeek-V3 gate/up and 7 % on its down projection).
static GemmPlan plan_for(int dtype, int64_t max_rows, int G, int d, int F) {
  if (dtype == MOE_F32) return {64, 3};
  const double avg = (double)max_rows / (double)(G > 0 ? G : 1);
  if (avg >= 192.0) return {MOE_CFG0_BM, 0};
  if (avg >= 48.0 || F % 256 != 0 || d % 256 != 0) return {256, 1};
  return {32, 2};
}

// Medium-plan projections with bf16 weights and a long reduction (K >= 4096,
// 64 or more 64-K stages) run on the ping-pong kernel: the medium tiles' work
// lists (256-row M-tiles, 128 gate/up and 256 down columns) are the
// ping-pong kernel's, and with the rows of a ~128-row tile split 64 + 64
// between its wave groups it streams the weights faster there (same GPU,
// alternating builds: DeepSeek-V3 gate/up, K = 7168, 2991 -> 2863 us;
// Switch down, K = 4096, 110 -> 109 us).  With K = 2048 its prologue and
// epilogue weigh more and the four-wave kernel stays (DeepSeek-V3 down
// 1879 us against 1935, Switch gate/up 240 against 249), and so it does for
// FP8 weights, where the ping-pong kernel was slower on both shapes
// (DeepSeek-V3 gate/up 2456 -> 2686 us, Switch down 92 -> 103 us).
static bool medium_on_pp(int K) { return K >= 4096; }

static int num_cus();

// Upper bound of work entries for one projection with N-tile width BN (a
// K-split of the last tiles adds at most one dispatch round of entries).
static int64_t max_work(int64_t max_rows, int G, int BM, int N, int BN, int tail = 1) {
  return (MOE_CEIL_DIV(max_rows, BM) + G) * (int64_t)(N / BN) +
         (tail > 1 ? (num_cus() & ~7) : 0);
}

// N-tile widths: gate/up tiles hold 128 columns of h (256 weight rows);
// down tiles 256 columns of y for the large and medium shapes, 128 for the
// decode and fp32 shapes (narrower decode tiles give more blocks to stream
// the weights: -2 % on bf16 and -6 % on FP8 decode gate/up).
static int up_bn(int) { return 128; }
static int down_bn(int cfg, int d) { return (cfg == 2 || cfg == 3 || d % 256 != 0) ? 128 : 256; }

// Largest K-split of the down projection's last tiles (large tiles, 256
// columns: the ping-pong kernel).  The tiles after the last full dispatch
// round would otherwise leave most CUs idle for a whole tile (Mixtral-shaped
// layer: 576 tiles, 2.25 rounds of 256 CUs); split 2^lg ways they take
// 1 / 2^lg of a tile.  Each part keeps at least 1024 of K (16 stages).
static int down_tail(const GemmPlan& p, int d, int F) {
  if (p.cfg != 0 || down_bn(p.cfg, d) != 256) return 1;
  int t = 1;
  while (t < 8 && F % (128 * t) == 0 && F / (2 * t) >= 1024) t *= 2;
  return t;
}

// Workspace of the split tiles: partial tiles of BM x BN floats, one per
// part; at most one dispatch round of parts, and at most `tail` parts per
// tile the list can hold (few-tile shapes need few slots).
static size_t tail_ws_bytes(int tail, int64_t max_rows, int G, int d) {
  if (tail <= 1) return 0;
  const int64_t tiles = max_work(max_rows, G, PPRing::BM, d, PPRing::BN);
  const int64_t slots = std::min<int64_t>(num_cus() & ~7, tiles * tail);
  return (size_t)slots * PPRing::BM * PPRing::BN * sizeof(float);
}

// Tile height the work lists are sized for (one plan serves bf16 and FP8
// weights, so one workspace size serves both).
static int ws_tile_rows(int dtype, int64_t max_rows, int G, int d, int F) {
  return plan_for(dtype, max_rows, G, d, F).BM;
}

size_t ffn_ws_bytes(int64_t max_rows, int G, int d, int F, int dtype) {
  const int es = dtype == MOE_BF16 ? 2 : 4;
  const GemmPlan p = plan_for(dtype, max_rows, G, d, F);
  const int bm = ws_tile_rows(dtype, max_rows, G, d, F);
  const int tail = down_tail(p, d, F);
  const int64_t wu = max_work(max_rows, G, bm, F, up_bn(p.cfg));
  const int64_t wd = max_work(max_rows, G, bm, d, down_bn(p.cfg, d), tail);
  size_t b = align256((size_t)max_rows * F * es);                       // H
  b += align256((size_t)wu * sizeof(int2)) + align256((size_t)wd * sizeof(int2));  // work lists
  b += align256(4 * sizeof(int32_t));                                  // entry counts
  b += align256((size_t)(G + 1) * sizeof(int32_t));                    // group bounds
  b += tail_ws_bytes(tail, max_rows, G, d);                           // split tiles
  return b;
}

static int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

struct GemmArgs {
  const void* A;
  const int32_t* row_token;
  const int32_t* offsets;
  int G;
  const void *B0, *B1, *B0l, *B1l;
  int g_last, K, N, max_rows;
  void* out;
  int2* work;
  int32_t* nwork;
  int ksplit;                             // dense products: K-splits
  float* out2;                            // dense: the other splits; list: split tiles
  const float *sc0, *sc1, *sc0l, *sc1l;   // FP8 weights: per-output-channel scales
  int tail = 1;                           // list: largest K-split of the last tiles
};

static WorkListArgs work_list_args(const GemmArgs& a, int BM, int BN, bool glu) {
  const int NN = a.N / BN;
  const int NG = glu ? 8 : 4;
  return WorkListArgs{BM, NN, NG < NN ? NG : NN, a.tail, num_cus() & ~7, a.work, a.nwork};
}

// Builds the work list of a (and of b when given: same groups and offsets).
// `clean` receives the non-decreasing group bounds both GEMMs then read.
static void run_work_list(const GemmArgs& a, const int32_t* offsets, int32_t* clean, int BM,
                          int BN, bool glu, hipStream_t s, const GemmArgs* b = nullptr,
                          int BMb = 0, int BNb = 0, bool glub = false) {
  const WorkListArgs l0 = work_list_args(a, BM, BN, glu);
  const WorkListArgs l1 = b ? work_list_args(*b, BMb, BNb, glub) : l0;
  hipLaunchKernelGGL(k_work_list, dim3(kWorkSlices, b ? 2 : 1), dim3(1024), 0, s, offsets, a.G,
                     a.max_rows, l0, l1, clean);
}

template <typename T, int BM, int BN, int WM, int WN, bool GLU>
static void run_gemm(const GemmArgs& a, hipStream_t s) {
  const int64_t ub = max_work(a.max_rows, a.G, BM, a.N, BN);
  const int round = num_cus() & ~7;           // blocks per dispatch round, whole XCDs
  const int64_t nb = MOE_CEIL_DIV(ub, round) * round;
  hipLaunchKernelGGL((k_moe_gemm<T, BM, BN, WM, WN, GLU>), dim3((unsigned)nb), dim3(kThreads), 0,
                     s, (const T*)a.A, a.row_token, a.offsets, a.work, a.nwork, (const T*)a.B0,
                     (const T*)a.B1, (const T*)a.B0l, (const T*)a.B1l, a.g_last, a.K, a.N,
                     a.max_rows, a.ksplit, round, a.out, a.out2);
}

template <bool GLU, bool BUF, bool Q8 = false>
static void run_pp(const GemmArgs& a, hipStream_t s) {
  const int64_t ub =
      max_work(a.max_rows, a.G, PPRing::BM, a.N, GLU ? PPRing::BN / 2 : PPRing::BN, a.tail);
  const int round = num_cus() & ~7;
  const int64_t nb = MOE_CEIL_DIV(ub, round) * round;
  hipLaunchKernelGGL((k_moe_pp<GLU, BUF, Q8>), dim3((unsigned)nb), dim3(512), 0, s,
                     (const uint16_t*)a.A, a.row_token, a.offsets, a.work, a.nwork, a.B0, a.B1,
                     a.B0l, a.B1l, a.g_last, a.K, a.N, a.max_rows, round, a.out, a.out2, a.sc0,
                     a.sc1, a.sc0l, a.sc1l);
}

template <int BM, int BN, int WM, int WN, bool GLU, int KB = 128, int NBUF = 2, bool Q8 = false,
          int NBB = NBUF, bool DENSE = false>
static void run_gemm_dma(const GemmArgs& a, hipStream_t s) {
  const int64_t ub = max_work(a.max_rows, a.G, BM, a.N, BN) * a.ksplit;   // dense: K-splits
  const int round = num_cus() & ~7;
  const int64_t nb = MOE_CEIL_DIV(ub, round) * round;
  using T = uint16_t;
  hipLaunchKernelGGL((k_moe_gemm_dma<BM, BN, WM, WN, GLU, KB, NBUF, Q8, NBB, DENSE>), dim3((unsigned)nb),
                     dim3(kThreads), 0, s, (const T*)a.A, a.row_token, a.offsets, a.work, a.nwork,
                     a.B0, a.B1, a.B0l, a.B1l, a.g_last, a.K, a.N, a.max_rows, a.ksplit, round,
                     a.out, a.out2, a.sc0, a.sc1, a.sc0l, a.sc1l);
}

// Adds up the parts of the down tiles the work list split along K.
static void run_tail_sum(const GemmArgs& a, hipStream_t s) {
  if (a.tail <= 1) return;
  const int round = num_cus() & ~7;
  hipLaunchKernelGGL(k_tail_sum, dim3((unsigned)(round / 2 * 8)), dim3(256), 0, s, a.work, a.nwork,
                     a.offsets, a.max_rows, a.N, a.out2, (float*)a.out);
}

// ---------------------------------------------------------------- router
// Router logits through the same tiled kernel, as a dense product (no work
// list, no group offsets): part[z][t][e] = sum over K-split z of X[t] . Wg[e].
// Used when E is a multiple of 64; the select kernel sums the splits in order.

static int router_bn(int E) { return E % 256 == 0 ? 256 : E % 128 == 0 ? 128 : 64; }

bool router_gemm_ok(int dtype, int64_t T, int d, int E, int split) {
  // row offsets inside the kernel are 32-bit element offsets: T * d < 2^31
  return dtype == MOE_BF16 && T >= 256 && T * (int64_t)d < ((int64_t)1 << 31) && E % 64 == 0 &&
         E / 64 < 16384 && split >= 1 && split < 256 && d % split == 0 && (d / split) % 128 == 0;
}

int router_gemm_tiles(int64_t T, int E) { return (int)MOE_CEIL_DIV(T, 128) * (E / router_bn(E)); }

size_t router_gemm_ws_bytes(int64_t, int, int, int) { return 0; }   // nothing beyond the partials

hipError_t launch_router_gemm(const void* X, const void* Wg, int64_t T, int d, int E, int split,
                              float* part, void* ws, hipStream_t s) {
  (void)ws;                    // a dense product: the kernel derives its tiles, no list
  const int bn = router_bn(E);
  const int mr = (int)T;
  GemmArgs a{X, nullptr, nullptr, 1, Wg, nullptr, nullptr, nullptr, -1, d, E, mr, part, nullptr,
             nullptr, split, part + (size_t)T * E};
  if (bn == 256) run_gemm_dma<128, 256, 2, 2, false, 128, 3, false, 3, true>(a, s);
  else if (bn == 128) run_gemm_dma<128, 128, 2, 2, false, 128, 3, false, 3, true>(a, s);
  else run_gemm_dma<128, 64, 2, 2, false, 128, 3, false, 3, true>(a, s);
  return hipGetLastError();
}

// rows x K elements of es bytes lie within 2^32 bytes of their base, so the
// buffer-form copies reach every one of them (rows < 0: not known).
static bool buf_fits(int64_t rows, int64_t K, int es) {
  return rows >= 0 && rows * K * es < ((int64_t)1 << 32);
}

// Runs both projections.  Groups [0, G) use W1/W3/W2 + g * stride; if
// g_last >= 0, group g_last uses the separate (shared-expert) matrices.
// Yrows receives the down projection (tiles split along K are summed by
// k_tail_sum before this returns to the stream's next launch).
hipError_t launch_grouped_ffn(const void* A, const int32_t* row_token, const int32_t* offsets,
                              int G, const void* W1, const void* W3, const void* W2,
                              const void* W1l, const void* W3l, const void* W2l, int g_last,
                              int dtype, int d, int F, int64_t max_rows, float* Yrows, void* ws,
                              hipStream_t s, const WeightScales* qs, int64_t a_rows) {
  if (max_rows <= 0 || G <= 0) return hipSuccess;
  const GemmPlan p = plan_for(dtype, max_rows, G, d, F);
  const int tail = down_tail(p, d, F);
  const int es = dtype == MOE_BF16 ? 2 : 4;
  // work-list regions laid out as in ffn_ws_bytes
  const int bm = ws_tile_rows(dtype, max_rows, G, d, F);
  const int64_t wu = max_work(max_rows, G, bm, F, up_bn(p.cfg));
  const int64_t wd = max_work(max_rows, G, bm, d, down_bn(p.cfg, d), tail);
  char* q = (char*)ws;
  void* H = q;               q += align256((size_t)max_rows * F * es);
  int2* work_up = (int2*)q;  q += align256((size_t)wu * sizeof(int2));
  int2* work_dn = (int2*)q;  q += align256((size_t)wd * sizeof(int2));
  int32_t* nwork = (int32_t*)q; q += align256(4 * sizeof(int32_t));   // two per list
  int32_t* bounds = (int32_t*)q; q += align256((size_t)(G + 1) * sizeof(int32_t));
  float* fix = tail > 1 ? (float*)q : nullptr;                        // split tiles
  const int mr = (int)max_rows;
  GemmArgs up{A,  row_token, bounds, G, W1, W3, W1l, W3l, g_last, d, F, mr, H, work_up, nwork,
              1,  nullptr};
  GemmArgs dn{H,  nullptr, bounds, G, W2, nullptr, W2l, nullptr, g_last, F, d, mr, Yrows, work_dn,
              nwork + 2, 1, fix};
  dn.tail = tail;
  if (qs) {
    up.sc0 = qs->s1; up.sc1 = qs->s3; up.sc0l = qs->s1l; up.sc1l = qs->s3l;
    dn.sc0 = qs->s2; dn.sc0l = qs->s2l;
  }
  run_work_list(up, offsets, bounds, p.BM, up_bn(p.cfg), true, s, &dn, p.BM, down_bn(p.cfg, d),
                false);
  timing_mark("tile_map", s);
  if (qs) {
    // FP8 weights: the large and medium tiles keep 64-K stages (32 KB of A
    // rows and 16 KB of weight codes per stage; three code buffers); decode
    // tiles use 128-K stages (256-B A rows, 128-B weight rows: whole cache
    // lines per copy).
    switch (p.cfg) {
      case 0:
        if (buf_fits(a_rows, d, 2) && buf_fits(F, d, 1)) run_pp<true, true, true>(up, s);
        else run_pp<true, false, true>(up, s);
        break;
      case 1: run_gemm_dma<256, 128, 1, 4, true, 128, 2, true, 3>(up, s); break;
      default: run_gemm_dma<32, 128, 1, 4, true, 256, 2, true>(up, s); break;
    }
    timing_mark("ffn_up", s);
    const bool b256 = down_bn(p.cfg, d) == 256;
    switch (p.cfg) {
      case 0:
        if (b256 && buf_fits(max_rows, F, 2) && buf_fits(d, F, 1)) run_pp<false, true, true>(dn, s);
        else if (b256) run_pp<false, false, true>(dn, s);
        else run_gemm_dma<MOE_CFG0_BM, 128, 2, 2, false, 128, 2, true>(dn, s);
        break;
      case 1:
        if (b256) run_gemm_dma<256, 256, 1, 4, false, 128, 2, true, 3>(dn, s);
        else run_gemm_dma<256, 128, 1, 4, false, 128, 2, true, 3>(dn, s);
        break;
      default: run_gemm_dma<32, 128, 1, 4, false, 256, 2, true>(dn, s); break;
    }
    run_tail_sum(dn, s);
    timing_mark("ffn_down", s);
  } else if (dtype == MOE_BF16) {
    using T = uint16_t;
    switch (p.cfg) {
      case 0:
        if (buf_fits(a_rows, d, 2) && buf_fits(F, d, 2)) run_pp<true, true>(up, s);
        else run_pp<true, false>(up, s);
        break;
      case 1:
        if (!medium_on_pp(d)) run_gemm_dma<256, 128, 1, 4, true, 128, 2, false, 3>(up, s);
        else if (buf_fits(a_rows, d, 2) && buf_fits(F, d, 2)) run_pp<true, true>(up, s);
        else run_pp<true, false>(up, s);
        break;
      default: run_gemm<T, 32, 128, 1, 4, true>(up, s); break;
    }
    timing_mark("ffn_up", s);
    const bool b256 = down_bn(p.cfg, d) == 256;
    switch (p.cfg) {
      case 0:
        if (b256 && buf_fits(max_rows, F, 2) && buf_fits(d, F, 2)) run_pp<false, true>(dn, s);
        else if (b256) run_pp<false, false>(dn, s);
        else run_gemm_dma<MOE_CFG0_BM, 128, 2, 2, false, 128, 2, false, MOE_CFG0_NBB>(dn, s);
        break;
      case 1:
        if (b256 && medium_on_pp(F) && buf_fits(max_rows, F, 2) && buf_fits(d, F, 2))
          run_pp<false, true>(dn, s);
        else if (b256 && medium_on_pp(F)) run_pp<false, false>(dn, s);
        else if (b256) run_gemm_dma<256, 256, 1, 4, false, 128, 2, false, 3>(dn, s);
        else run_gemm_dma<256, 128, 1, 4, false, 128, 2, false, 3>(dn, s);
        break;
      default: run_gemm<T, 32, 128, 1, 4, false>(dn, s); break;
    }
    run_tail_sum(dn, s);
    timing_mark("ffn_down", s);
  } else {
    run_gemm<float, 64, 128, 2, 2, true>(up, s);
    timing_mark("ffn_up", s);
    run_gemm<float, 64, 128, 2, 2, false>(dn, s);
    timing_mark("ffn_down", s);
  }
  return hipGetLastError();
}

}  // namespace moe
