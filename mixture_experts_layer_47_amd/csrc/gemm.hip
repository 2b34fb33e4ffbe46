// Grouped expert GEMMs on CDNA4 matrix cores.
//
// LLM Internals 14.2.1 step 5: every expert multiplies its own m_i rows,
// [m_i, d] x W_i[d, F] -> [m_i, F], then projects back to d; the row counts
// differ per expert.  One expert is a SwiGLU block of three matrices
// (14.2.2): h = silu(x W1) * (x W3), y = h W2.
//
// Kernel shape (one launch per projection):
//   * a device-built tile list maps each M-tile to (expert g, first row);
//     the grid is sized from host bounds only, surplus blocks exit at once;
//   * block tile BM x BNT, BK = 128 bytes of K per stage (64 bf16 / 32 fp32),
//     two LDS stages filled through registers while the other is consumed;
//   * LDS rows are 8 chunks of 16 B, chunk index XOR (row & 7) so both the
//     16-B stores and the MFMA fragment loads are bank-conflict free;
//   * bf16: v_mfma_f32_32x32x16_bf16, each lane feeds 8 K-contiguous values
//     per operand; fp32: four v_mfma_f32_32x32x2f32 per 16-B fragment;
//   * gate/up fusion: the B tile holds BN rows of W1 then BN rows of W3, a
//     wave owns matching gate and up columns, and SwiGLU runs on the fp32
//     accumulators before one rounding of h to the storage type;
//   * XCD-aware order: consecutive logical tiles (same weight slice,
//     neighbouring M-tiles) land on the same XCD and share its L2.
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
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[i]), __uint_as_float(b[i]), acc, 0, 0, 0);
  }
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.f + __expf(-x)); }

template <typename T>
__device__ __forceinline__ void store_h(T* p, float v);
template <>
__device__ __forceinline__ void store_h<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
template <>
__device__ __forceinline__ void store_h<float>(float* p, float v) { *p = v; }

// Global -> registers for one K stage (k0 = first element of the stage).
template <typename T, int CA, int CB, bool GLU, int BN, int NT>
__device__ __forceinline__ void gload_tile(u32x4 (&ra)[CA], u32x4 (&rb)[CB], const T* A,
                                           const uint32_t (&oa)[CA], uint32_t vmask,
                                           const T* pb0, const T* pb1, size_t bstep, bool bact,
                                           int k0) {
  const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < CA; ++i)
    ra[i] = ((vmask >> i) & 1u) ? *(const u32x4*)(A + oa[i] + k0) : z4;
  if (bact) {
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      constexpr int kSplit = BN / (NT / 8);     // first thread-row index in the W3 half
      const T* p = (GLU && i >= kSplit) ? pb1 + (size_t)(i - kSplit) * bstep
                                        : pb0 + (size_t)i * bstep;
      rb[i] = *(const u32x4*)(p + k0);
    }
  }
}

// Registers -> one LDS stage; chunk c of row r lands in slot c ^ (r & 7).
template <int BM, int CA, int CB, int NT>
__device__ __forceinline__ void lstore_tile(u32x4* sm, const u32x4 (&ra)[CA],
                                            const u32x4 (&rb)[CB], int tid, int c16, bool ast,
                                            bool bact) {
  if (ast) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int r = (tid >> 3) + i * (NT / 8);
      sm[r * 8 + (c16 ^ (r & 7))] = ra[i];
    }
  }
  if (bact) {
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int r = BM + (tid >> 3) + i * (NT / 8);
      sm[r * 8 + (c16 ^ (r & 7))] = rb[i];
    }
  }
}

// GLU = true : out = H [rows][N] (type T),  h = silu(A W1^T) * (A W3^T)
// GLU = false: out = Y [rows][N] (fp32),    y = A W2^T
template <typename T, int BM, int BN, int WM, int WN, bool GLU>
__global__ __launch_bounds__(WM * WN * 64) void k_grouped_gemm(
    const T* __restrict__ A, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const int2* __restrict__ tiles,
    const int32_t* __restrict__ ntiles, const T* __restrict__ B0, const T* __restrict__ B1,
    const T* __restrict__ B0_last, const T* __restrict__ B1_last, int g_last, int K, int N,
    int MT, int max_rows, void* __restrict__ out) {
  constexpr int NT = WM * WN * 64;
  constexpr int BNT = GLU ? 2 * BN : BN;
  constexpr int EPC = 16 / sizeof(T);          // elements per 16-B chunk
  constexpr int BK = 8 * EPC;                  // elements per stage (128 B)
  // 16-B chunks per thread per stage; when a tile has fewer chunks than the
  // block has threads, only the first BM*8 (BNT*8) threads load.
  constexpr int CA = BM * 8 >= NT ? BM * 8 / NT : 1;
  constexpr int CB = BNT * 8 >= NT ? BNT * 8 / NT : 1;
  constexpr bool PA = BM * 8 < NT, PB = BNT * 8 < NT;
  constexpr int WROWS = BM / WM, WCOLS = BNT / WN;
  constexpr int FM = WROWS / 32, FN = WCOLS / 32;
  constexpr int FNH = GLU ? FN / 2 : FN;
  static_assert((BM * 8) % NT == 0 || NT % (BM * 8) == 0, "A tile vs threads");
  static_assert((BNT * 8) % NT == 0 || NT % (BNT * 8) == 0, "B tile vs threads");
  static_assert(FM >= 1 && FN >= 1 && (!GLU || FN % 2 == 0), "wave tile");
  static_assert(!GLU || (!PB && BN % (NT / 8) == 0), "gate/up halves split on thread rows");
  __shared__ u32x4 smem[2][(BM + BNT) * 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = xcd_swizzle(blockIdx.x, gridDim.x);
  const int n_idx = L / MT, m_idx = L - n_idx * MT;
  if (m_idx >= ntiles[0]) return;
  const int2 tl = tiles[m_idx];
  const int g = tl.x;
  const int gbeg = min(max(offsets[g], 0), max_rows);
  const int rbeg = gbeg + tl.y;
  const int rows = min(BM, min(max(offsets[g + 1], gbeg), max_rows) - rbeg);
  const int n0 = n_idx * BN;

  const T* w0 = (g == g_last) ? B0_last : B0 + (size_t)g * N * K;
  const T* w1 = GLU ? ((g == g_last) ? B1_last : B1 + (size_t)g * N * K) : nullptr;

  // ---- per-thread global source rows (fixed for the whole K loop), kept as
  // 32-bit element offsets (every operand here holds < 2^31 elements)
  const int c16 = tid & 7;                     // 16-B chunk inside the 128-B row
  uint32_t oa[CA];
  uint32_t vmask = 0;
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int r = (tid >> 3) + i * (NT / 8);
    const bool v = r < rows && (!PA || tid < BM * 8);
    int src = rbeg + (v ? r : 0);
    if (row_token) src = row_token[src];
    oa[i] = (uint32_t)src * (uint32_t)K + c16 * EPC;
    vmask |= (v ? 1u : 0u) << i;
  }
  // B rows: thread row r0 = tid/8 + i*NT/8; GLU tiles take W1 rows then W3 rows.
  const bool bact = !PB || tid < BNT * 8;
  const T* pb0;
  const T* pb1 = nullptr;                      // W3 half (GLU only)
  {
    const int r0 = bact ? (tid >> 3) : 0;
    pb0 = w0 + (size_t)(n0 + r0) * K + c16 * EPC;
    if constexpr (GLU) pb1 = w1 + (size_t)(n0 + r0) * K + c16 * EPC;
  }
  const size_t bstep = (size_t)(NT / 8) * K;   // element distance between a thread's B rows

  u32x4 ra[CA], rb[CB];
  const int wm = wave / WN, wn = wave % WN;
  const int arow0 = wm * WROWS;                // wave's first A row in the tile
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS row of the wave's j-th B fragment (lane's column = lane & 31).
#define MOE_BROW(j)                                                                 \
  (GLU ? BM + (((j) < FNH) ? wn * (BN / WN) + (j) * 32                             \
                           : BN + wn * (BN / WN) + ((j) - FNH) * 32) + (lane & 31) \
       : BM + wn * WCOLS + (j) * 32 + (lane & 31))

  const int nk = K / BK;
  const bool ast = !PA || tid < BM * 8;
  gload_tile<T, CA, CB, GLU, BN, NT>(ra, rb, A, oa, vmask, pb0, pb1, bstep, bact, 0);
  lstore_tile<BM, CA, CB, NT>(smem[0], ra, rb, tid, c16, ast, bact);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk)
      gload_tile<T, CA, CB, GLU, BN, NT>(ra, rb, A, oa, vmask, pb0, pb1, bstep, bact, (kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kc = 2 * s + (lane >> 5);
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = arow0 + i * 32 + (lane & 31);
        af[i] = smem[buf][r * 8 + (kc ^ (r & 7))];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = MOE_BROW(j);
        bfr[j] = smem[buf][r * 8 + (kc ^ (r & 7))];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma_32x32<T>(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < nk) lstore_tile<BM, CA, CB, NT>(smem[buf ^ 1], ra, rb, tid, c16, ast, bact);
    __syncthreads();
  }

#undef MOE_BROW
  // ---- epilogue.  32x32 C layout: lane holds column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + (r%4) for r = 0..15.
  const int col_l = lane & 31;
  const int rsub = (lane >> 5) * 4;
  if constexpr (GLU) {
    T* H = (T*)out;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FNH; ++j) {
        const int col = n0 + wn * (BN / WN) + j * 32 + col_l;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = arow0 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          if (row < rows) {
            const float h = silu_f(acc[i][j][r]) * acc[i][j + FNH][r];
            store_h<T>(H + (size_t)(rbeg + row) * N + col, h);
          }
        }
      }
  } else {
    float* Y = (float*)out;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WCOLS + j * 32 + col_l;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = arow0 + i * 32 + (r >> 2) * 8 + rsub + (r & 3);
          if (row < rows) Y[(size_t)(rbeg + row) * N + col] = acc[i][j][r];
        }
      }
  }
}

// Tile list: for group g, ceil(rows_g / BM) tiles (g, i*BM).  One block.
// Group row ranges are clamped to [0, max_rows), so malformed offsets can
// never address rows outside the caller's buffers.
__global__ __launch_bounds__(1024) void k_tile_map(const int32_t* __restrict__ offsets, int G,
                                                   int BM, int max_rows, int2* __restrict__ tiles,
                                                   int32_t* __restrict__ ntiles) {
  __shared__ int32_t sc[1024];
  const int g = threadIdx.x;
  int nt = 0;
  if (g < G) {
    const int a = min(max(offsets[g], 0), max_rows);
    const int b = min(max(offsets[g + 1], a), max_rows);
    nt = MOE_CEIL_DIV(b - a, BM);
  }
  sc[g] = nt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {       // inclusive Hillis-Steele scan
    const int v = (g >= o) ? sc[g - o] : 0;
    __syncthreads();
    sc[g] += v;
    __syncthreads();
  }
  const int start = sc[g] - nt;        // total <= ceil(max_rows / BM) + G
  for (int i = 0; i < nt; ++i) tiles[start + i] = make_int2(g, i * BM);
  if (g == 1023) ntiles[0] = sc[1023];
}

// ------------------------------------------------------------------ launch
struct GemmPlan {
  int BM;
  int cfg;   // 0 = large, 1 = medium, 2 = small (decode), 3 = fp32
};

static GemmPlan plan_for(int dtype, int64_t max_rows, int G, int d, int F) {
  if (dtype == MOE_F32) return {64, 3};
  const double avg = (double)max_rows / (double)(G > 0 ? G : 1);
  if (avg >= 192.0) return {256, 0};
  if (avg >= 48.0 || F % 256 != 0 || d % 256 != 0) return {128, 1};
  return {32, 2};
}

int64_t gemm_max_mtiles(int64_t max_rows, int G, int BM) {
  return MOE_CEIL_DIV(max_rows, BM) + G;
}

size_t ffn_ws_bytes(int64_t max_rows, int G, int d, int F, int dtype) {
  const int es = dtype == MOE_BF16 ? 2 : 4;
  const GemmPlan p = plan_for(dtype, max_rows, G, d, F);
  size_t b = align256((size_t)max_rows * F * es);                         // H
  b += align256((size_t)gemm_max_mtiles(max_rows, G, p.BM) * sizeof(int2));  // tiles
  b += align256(sizeof(int32_t));                                        // tile count
  return b;
}

template <typename T, int BM, int BN, int WM, int WN, bool GLU>
static void run_gemm(const T* A, const int32_t* row_token, const int32_t* offsets,
                     const int2* tiles, const int32_t* ntiles, const T* B0, const T* B1,
                     const T* B0l, const T* B1l, int g_last, int K, int N, int MT, int max_rows,
                     void* out, hipStream_t s) {
  const int nn = N / BN;
  const unsigned grid = (unsigned)((int64_t)nn * MT);
  hipLaunchKernelGGL((k_grouped_gemm<T, BM, BN, WM, WN, GLU>), dim3(grid), dim3(WM * WN * 64), 0,
                     s, A, row_token, offsets, tiles, ntiles, B0, B1, B0l, B1l, g_last, K, N, MT,
                     max_rows, out);
}

template <typename T>
static void run_up_bf16(int cfg, const T* A, const int32_t* rt, const int32_t* off, const int2* tl,
                   const int32_t* nt, const T* W1, const T* W3, const T* W1l, const T* W3l,
                   int gl, int d, int F, int MT, int mr, T* H, hipStream_t s) {
  switch (cfg) {
    case 0: run_gemm<T, 256, 128, 4, 2, true>(A, rt, off, tl, nt, W1, W3, W1l, W3l, gl, d, F, MT, mr, H, s); break;
    case 1: run_gemm<T, 128, 128, 2, 4, true>(A, rt, off, tl, nt, W1, W3, W1l, W3l, gl, d, F, MT, mr, H, s); break;
    default: run_gemm<T, 32, 256, 1, 8, true>(A, rt, off, tl, nt, W1, W3, W1l, W3l, gl, d, F, MT, mr, H, s); break;
  }
}

template <typename T>
static void run_down_bf16(int cfg, const T* H, const int32_t* off, const int2* tl, const int32_t* nt,
                     const T* W2, const T* W2l, int gl, int d, int F, int MT, int mr,
                     float* Y, hipStream_t s) {
  const bool b256 = d % 256 == 0;
  switch (cfg) {
    case 0:
      if (b256) run_gemm<T, 256, 256, 4, 2, false>(H, nullptr, off, tl, nt, W2, nullptr, W2l, nullptr, gl, F, d, MT, mr, Y, s);
      else      run_gemm<T, 256, 128, 4, 2, false>(H, nullptr, off, tl, nt, W2, nullptr, W2l, nullptr, gl, F, d, MT, mr, Y, s);
      break;
    case 1:
      if (b256) run_gemm<T, 128, 256, 2, 4, false>(H, nullptr, off, tl, nt, W2, nullptr, W2l, nullptr, gl, F, d, MT, mr, Y, s);
      else      run_gemm<T, 128, 128, 2, 4, false>(H, nullptr, off, tl, nt, W2, nullptr, W2l, nullptr, gl, F, d, MT, mr, Y, s);
      break;
    default:
      run_gemm<T, 32, 256, 1, 8, false>(H, nullptr, off, tl, nt, W2, nullptr, W2l, nullptr, gl, F, d, MT, mr, Y, s);
      break;
  }
}

// Runs both projections.  Groups [0, G) use W1/W3/W2 + g * stride; if
// g_last >= 0, group g_last uses the separate (shared-expert) matrices.
hipError_t launch_grouped_ffn(const void* A, const int32_t* row_token, const int32_t* offsets,
                              int G, const void* W1, const void* W3, const void* W2,
                              const void* W1l, const void* W3l, const void* W2l, int g_last,
                              int dtype, int d, int F, int64_t max_rows, float* Yrows, void* ws,
                              hipStream_t s) {
  if (max_rows <= 0 || G <= 0) return hipSuccess;
  const GemmPlan p = plan_for(dtype, max_rows, G, d, F);
  const int es = dtype == MOE_BF16 ? 2 : 4;
  char* q = (char*)ws;
  void* H = q;             q += align256((size_t)max_rows * F * es);
  const int64_t MT = gemm_max_mtiles(max_rows, G, p.BM);
  int2* tiles = (int2*)q;  q += align256((size_t)MT * sizeof(int2));
  int32_t* ntiles = (int32_t*)q;
  const int mr = (int)max_rows;
  hipLaunchKernelGGL(k_tile_map, dim3(1), dim3(1024), 0, s, offsets, G, p.BM, mr, tiles, ntiles);
  timing_mark("tile_map", s);
  if (dtype == MOE_BF16) {
    using T = uint16_t;
    run_up_bf16<T>(p.cfg, (const T*)A, row_token, offsets, tiles, ntiles, (const T*)W1, (const T*)W3,
              (const T*)W1l, (const T*)W3l, g_last, d, F, (int)MT, mr, (T*)H, s);
    timing_mark("ffn_up", s);
    run_down_bf16<T>(p.cfg, (const T*)H, offsets, tiles, ntiles, (const T*)W2, (const T*)W2l,
                     g_last, d, F, (int)MT, mr, Yrows, s);
    timing_mark("ffn_down", s);
  } else {
    using T = float;
    run_gemm<T, 64, 128, 2, 4, true>((const T*)A, row_token, offsets, tiles, ntiles, (const T*)W1,
                                     (const T*)W3, (const T*)W1l, (const T*)W3l, g_last, d, F,
                                     (int)MT, mr, H, s);
    timing_mark("ffn_up", s);
    run_gemm<T, 64, 128, 2, 4, false>((const T*)H, nullptr, offsets, tiles, ntiles, (const T*)W2,
                                      nullptr, (const T*)W2l, nullptr, g_last, F, d, (int)MT,
                                      mr, Yrows, s);
    timing_mark("ffn_down", s);
  }
  return hipGetLastError();
}

}  // namespace moe
