// Dispatch ("moe_align"): per-expert histogram, exclusive scan, stable rank,
// capacity drop, and the expert-sorted permutation; plus the row gather.
//
// LLM Internals 14.2.1 step 4 (sort token slots by expert so each expert's
// rows are contiguous; steps 4 and 6 are mutually inverse permutations) and
// the AI Knowledge Map "MoE" capacity rule C = ceil(c N k / E) with overflow
// dropped.  Slot s = t*k + j keeps its place iff fewer than C earlier slots
// chose the same expert.
//
// Atomic-free: a wave walks a fixed chunk of slots 64 at a time; lanes that
// hold the same expert id find each other with one ballot per id bit (a wave
// "multisplit"), so in-wave ranks come from popcounts, and per-expert running
// counts live in the wave's own LDS row.  Results are identical run to run.
#include "common.h"
#include "kernels.h"

namespace moe {

// Slots per wave (chunk): 256, four groups of 64.  Short chunks give more
// waves; the per-expert walk over chunk histograms that grows with them
// keeps eight chunks' loads in flight (with 256 experts and 32768 slots,
// chunks of 256 measured 27 us against 31 us for 512 and 40 us for 1024).
__host__ __device__ constexpr int align_chunk_for(int) { return 256; }

// Mask of active lanes whose expert id equals this lane's.
__device__ __forceinline__ uint64_t match_id(int e, bool valid, int nbits) {
  uint64_t eq = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(valid && bit);
    eq &= bit ? bal : ~bal;
  }
  return valid ? eq : 0ull;
}

// Only ids in [0, E) take part in a dispatch; a slot holding any other value
// is left out of the counts and gets row -1 (it contributes nothing), so no
// index outside the per-expert tables is ever formed.
__device__ __forceinline__ bool id_ok(int e, int E) { return (unsigned)e < (unsigned)E; }

__device__ __forceinline__ int nbits_for(int E) {
  return E <= 1 ? 0 : 32 - __clz(E - 1);
}

// Expert e's column of the chunk histograms hist[c][e] becomes exclusive
// per-chunk bases (chunk order); returns the expert's total.  Eight chunks'
// loads are in flight at once.
__device__ __forceinline__ int chunk_bases(int32_t* __restrict__ hist, int E, int nchunks, int e) {
  int run = 0, c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    int h[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) h[u] = hist[(size_t)(c + u) * E + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      hist[(size_t)(c + u) * E + e] = run;
      run += h[u];
    }
  }
  for (; c < nchunks; ++c) {
    const int h = hist[(size_t)c * E + e];
    hist[(size_t)c * E + e] = run;
    run += h;
  }
  return run;
}

// Exclusive scan of the per-expert row counts in[0..E) (E <= 256, LDS) by
// one wave, four experts per lane: offsets[0..E], offsets[E + 1] = total +
// tail_rows when there is a tail, n_kept = total; out (LDS, may be in)
// receives the offsets and out[256] the total when given.
__device__ __forceinline__ void wave_offsets(const int32_t* in, int E, int tail_rows,
                                             int32_t* __restrict__ offsets,
                                             int32_t* __restrict__ n_kept, int32_t* out) {
  const int lane = threadIdx.x & 63;
  int v[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane * 4 + i;
    v[i] = e < E ? in[e] : 0;
    sum += v[i];
  }
  int inc = sum;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  int acc = inc - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane * 4 + i;
    if (e < E) {
      offsets[e] = acc;
      if (out) out[e] = acc;
    }
    acc += v[i];
  }
  if (lane == 63) {
    offsets[E] = acc;
    if (tail_rows > 0) offsets[E + 1] = acc + tail_rows;
    n_kept[0] = acc;
    if (out) out[256] = acc;
  }
}

// Pass 1: chunk histograms hist[c][e].
template <int CHUNK>
__global__ __launch_bounds__(256) void k_align_count(const int32_t* __restrict__ ids,
                                                     int64_t Tk, int E, int nchunks,
                                                     int32_t* __restrict__ hist) {
  __shared__ int32_t cnt_[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * 4 + wave;
  if (c >= nchunks) return;                           // no block sync below
  // Each wave owns one LDS row; volatile keeps its in-order LDS traffic as written.
  volatile int32_t* cnt = cnt_[wave];
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  const int nb = nbits_for(E);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int NG = CHUNK / 64;
  int ev[NG];                                         // all loads in flight at once
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int64_t s = (int64_t)c * CHUNK + g * 64 + lane;
    ev[g] = s < Tk ? ids[s] : -1;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const bool v = id_ok(ev[g], E);
    const int e = v ? ev[g] : 0;
    const uint64_t eq = match_id(e, v, nb);
    if (v && (eq & lt) == 0)                          // lowest lane of its id
      cnt[e] = cnt[e] + __popcll(eq);
  }
  for (int e = lane; e < E; e += 64) hist[(size_t)c * E + e] = cnt[e];
}

// Pass 2: per-expert chunk bases, counts, capacity, offsets.  One block.
// Thread e walks the chunks in order; experts are then scanned by the block.
__global__ __launch_bounds__(256) void k_align_scan(int32_t* __restrict__ hist, int E,
                                                    int nchunks, int64_t cap,
                                                    int tail_rows,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ n_kept) {
  __shared__ int32_t kept[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    run = chunk_bases(hist, E, nchunks, e);       // hist becomes exclusive bases
    counts[e] = run;
  }
  kept[e] = (e < E) ? (cap > 0 && run > cap ? (int)cap : run) : 0;
  __syncthreads();
  if (threadIdx.x < 64) wave_offsets(kept, E, tail_rows, offsets, n_kept, nullptr);
}

// Pass 3: stable ranks, drop mask and the permutation.
template <int CHUNK>
__global__ __launch_bounds__(256) void k_align_scatter(
    const int32_t* __restrict__ ids, int64_t Tk, int k, int E, int nchunks,
    int64_t cap, const int32_t* __restrict__ base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token) {
  __shared__ int32_t cnt_[4][256];
  __shared__ int32_t off[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 256) off[e] = offsets[e];
  __syncthreads();
  const int c = blockIdx.x * 4 + wave;
  if (c >= nchunks) return;
  volatile int32_t* cnt = cnt_[wave];
  for (int e = lane; e < E; e += 64) cnt[e] = base[(size_t)c * E + e];
  const int nb = nbits_for(E);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int NG = CHUNK / 64;
  int ev[NG];                                         // all loads in flight at once
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int64_t s = (int64_t)c * CHUNK + g * 64 + lane;
    ev[g] = s < Tk ? ids[s] : -1;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int64_t s = (int64_t)c * CHUNK + g * 64 + lane;
    const bool v = id_ok(ev[g], E);
    const int e = v ? ev[g] : 0;
    const uint64_t eq = match_id(e, v, nb);
    int rank = 0;
    if (v) rank = cnt[e] + __popcll(eq & lt);
    // every lane has read its base before any leader writes the update
    __builtin_amdgcn_wave_barrier();
    if (v && (eq & lt) == 0) cnt[e] = rank + __popcll(eq);
    if (v) {
      const bool keep = cap <= 0 || rank < cap;
      const int row = keep ? off[e] + rank : -1;
      slot_row[s] = row;
      if (keep) {
        sorted_slot[row] = (int32_t)s;
        if (row_token) row_token[row] = (int32_t)(s / k);
      }
    } else if (s < Tk) {
      slot_row[s] = -1;                               // id outside [0, E)
    }
  }
}

// ----------------------------------------------------------------------------
// Overflow re-route (AI Knowledge Map "MoE", capacity overflow handled by the
// second/backup option): one backup round after the capacity drop.  The m-th
// dropped slot of token t proposes the token's m-th backup expert; experts
// accept proposals in slot order while they have room; accepted slots are
// placed after the expert's first-pass rows.

// props[s]: the backup expert dropped slot s proposes, or -1.
// Slots whose own id lies outside [0, E) were never dispatched and propose
// nothing; a backup outside [0, E) is no proposal.
__global__ __launch_bounds__(256) void k_rr_props(const int32_t* __restrict__ ids,
                                                  const int32_t* __restrict__ slot_row,
                                                  const int32_t* __restrict__ backup,
                                                  int64_t T_, int k, int E, int nb,
                                                  int32_t* __restrict__ props) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T_) return;
  int m = 0;
  for (int j = 0; j < k; ++j) {
    const int64_t s = t * k + j;
    int p = -1;
    if (slot_row[s] < 0 && id_ok(ids[s], E)) {
      if (m < nb) p = backup[t * nb + m];
      if (!id_ok(p, E)) p = -1;
      ++m;
    }
    props[s] = p;
  }
}

// Proposal chunk bases (hist2 becomes exclusive), accepted proposals per
// expert, and the final offsets.  meta = {first-pass offsets, first-pass
// kept, accepted} x E.  One block, E <= 256.
__global__ __launch_bounds__(256) void k_rr_scan(int32_t* __restrict__ hist2, int E,
                                                 int nchunks, int64_t cap, int tail_rows,
                                                 const int32_t* __restrict__ counts,
                                                 int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ n_kept,
                                                 int32_t* __restrict__ meta) {
  __shared__ int32_t tot[256];
  const int e = threadIdx.x;
  if (e < E) {
    const int run = chunk_bases(hist2, E, nchunks, e);
    const int64_t kept1 = counts[e] < cap ? counts[e] : cap;
    const int64_t room = cap - kept1;
    const int acc = run < room ? run : (int)room;
    meta[e] = offsets[e];
    meta[E + e] = (int)kept1;
    meta[2 * E + e] = acc;
    tot[e] = (int)kept1 + acc;
  }
  __syncthreads();                                // old offsets read before the rewrite
  if (threadIdx.x < 64) wave_offsets(tot, E, tail_rows, offsets, n_kept, nullptr);
}

// Final placement of every slot: first-pass rows move by their expert's
// offset change; proposals are ranked in slot order (wave multisplit on
// the proposed expert, as in k_align_scatter) and placed after the
// expert's first-pass rows when the rank is below the accepted count.
template <int CHUNK>
__global__ __launch_bounds__(256) void k_rr_place(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ props, int64_t Tk, int k,
    int E, int nchunks, const int32_t* __restrict__ base2,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ meta,
    int32_t* __restrict__ sorted_slot, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token) {
  __shared__ int32_t cnt_[4][256];
  __shared__ int32_t off[256], off1[256], kept1[256], acc[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 256) {
    off[e] = offsets[e];
    off1[e] = meta[e];
    kept1[e] = meta[E + e];
    acc[e] = meta[2 * E + e];
  }
  __syncthreads();
  const int c = blockIdx.x * 4 + wave;
  if (c >= nchunks) return;
  volatile int32_t* cnt = cnt_[wave];
  for (int e = lane; e < E; e += 64) cnt[e] = base2[(size_t)c * E + e];
  const int nbits = nbits_for(E);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int NG = CHUNK / 64;
  for (int g = 0; g < NG; ++g) {
    const int64_t s = (int64_t)c * CHUNK + g * 64 + lane;
    const bool in = s < Tk;
    const int p = in ? props[s] : -1;
    const bool v = p >= 0;
    const int e = v ? p : 0;
    const uint64_t eq = match_id(e, v, nbits);
    int rank = 0;
    if (v) rank = cnt[e] + __popcll(eq & lt);
    __builtin_amdgcn_wave_barrier();
    if (v && (eq & lt) == 0) cnt[e] = rank + __popcll(eq);
    if (in) {
      int row = -1;
      if (v) {
        if (rank < acc[e]) row = off[e] + kept1[e] + rank;
      } else {
        const int r1 = slot_row[s];
        if (r1 >= 0) {
          const int e1 = ids[s];
          row = off[e1] + (r1 - off1[e1]);
        }
      }
      slot_row[s] = row;
      if (row >= 0) {
        sorted_slot[row] = (int32_t)s;
        if (row_token) row_token[row] = (int32_t)(s / k);
      }
    }
  }
}

// Few slots (at most 8192): the three passes in one block of 16 waves, with
// the chunk histograms, bases and offsets in LDS instead of global memory,
// and chunks of NG x 64 slots so that every wave has a chunk.  A stable rank
// does not depend on the chunking, so the ranks, drops and permutation are
// the same bits as the three-kernel path's; only launches and global round
// trips go away (decode batches).
constexpr int kSmallWaves = 16;
constexpr int64_t kSmallSlots = kSmallWaves * 8 * 64;
template <int NG>
__global__ __launch_bounds__(1024) void k_align_small(
    const int32_t* __restrict__ ids, int64_t Tk, int k, int E, int nchunks, int64_t cap,
    int tail_rows, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ n_kept, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ row_token) {
  __shared__ int32_t hist[kSmallWaves][256];
  __shared__ int32_t off[257];
  // The permutation (row -> slot) is built here and written out in row order
  // at the end: one CU storing it scattered, 4 B at a time, was the slowest
  // part of this kernel.
  __shared__ int32_t s_slot[kSmallSlots];
  const int lane = threadIdx.x & 63, c = threadIdx.x >> 6;
  const int nb = nbits_for(E);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int CHUNK = NG * 64;
  int ev[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int64_t sl = (int64_t)c * CHUNK + g * 64 + lane;
    ev[g] = (c < nchunks && sl < Tk) ? ids[sl] : -1;
  }
  // pass 1: chunk histograms
  volatile int32_t* cnt = hist[c];
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  if (c < nchunks) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const bool v = id_ok(ev[g], E);
      const int e = v ? ev[g] : 0;
      const uint64_t eq = match_id(e, v, nb);
      if (v && (eq & lt) == 0) cnt[e] = cnt[e] + __popcll(eq);
    }
  }
  __syncthreads();
  // pass 2: per-expert chunk bases, counts, kept rows; offsets by a wave scan
  int kept = 0;
  if (threadIdx.x < (unsigned)E) {
    const int e = threadIdx.x;
    int run = 0;
    for (int cc = 0; cc < nchunks; ++cc) {
      const int h = hist[cc][e];
      hist[cc][e] = run;
      run += h;
    }
    counts[e] = run;
    kept = (cap > 0 && run > cap) ? (int)cap : run;
    off[e] = kept;
  }
  __syncthreads();
  if (c == 0) wave_offsets(off, E, tail_rows, offsets, n_kept, off);
  __syncthreads();
  // pass 3: stable ranks, drops and the permutation
  if (c < nchunks) {
    volatile int32_t* base = hist[c];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int64_t sl = (int64_t)c * CHUNK + g * 64 + lane;
      const bool v = id_ok(ev[g], E);
      const int e = v ? ev[g] : 0;
      const uint64_t eq = match_id(e, v, nb);
      int rank = 0;
      if (v) rank = base[e] + __popcll(eq & lt);
      __builtin_amdgcn_wave_barrier();
      if (v && (eq & lt) == 0) base[e] = rank + __popcll(eq);
      if (v) {
        const bool keep = cap <= 0 || rank < cap;
        const int row = keep ? off[e] + rank : -1;
        slot_row[sl] = row;
        if (keep) s_slot[row] = (int32_t)sl;
      } else if (sl < Tk) {
        slot_row[sl] = -1;                            // id outside [0, E)
      }
    }
  }
  __syncthreads();
  const int nk = off[256];               // kept rows (<= Tk <= kSmallSlots)
  for (int r = threadIdx.x; r < nk; r += 1024) {
    const int32_t sl = s_slot[r];
    sorted_slot[r] = sl;
    if (row_token) row_token[r] = sl / k;
  }
  // shared-expert rows after the kept rows
  if (row_token)
    for (int t = threadIdx.x; t < tail_rows; t += 1024) row_token[nk + t] = t;
}

// Rows of the shared expert: row_token[R + t] = t, R read on the device.
__global__ __launch_bounds__(256) void k_tail_tokens(const int32_t* __restrict__ n_kept,
                                                     int T_, int32_t* __restrict__ row_token) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < T_) row_token[n_kept[0] + t] = t;
}

// Gather: Xs[r] = X[sorted_slot[r] / k] for r < n_kept.  16-B vectors.
__global__ __launch_bounds__(256) void k_gather_rows(const uint4* __restrict__ X,
                                                     const int32_t* __restrict__ sorted_slot,
                                                     const int32_t* __restrict__ n_kept,
                                                     int k, int vec_per_row,
                                                     uint4* __restrict__ Xs) {
  const int r = blockIdx.x;
  if (r >= n_kept[0]) return;
  const int t = sorted_slot[r] / k;
  const uint4* src = X + (size_t)t * vec_per_row;
  uint4* dst = Xs + (size_t)r * vec_per_row;
  for (int i = threadIdx.x; i < vec_per_row; i += 256) dst[i] = src[i];
}

__global__ void k_zero_words(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// --------------------------------------------------------------- launchers
int align_nchunks(int64_t Tk, int E) { return (int)MOE_CEIL_DIV(Tk, align_chunk_for(E)); }

size_t dispatch_ws_bytes(int64_t T, int k, int E) {
  const int64_t Tk = T * (int64_t)k;
  return align256((size_t)(align_nchunks(Tk, E) > 0 ? align_nchunks(Tk, E) : 1) * E * sizeof(int32_t));
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_words, dim3((unsigned)MOE_CEIL_DIV(n, 256)), dim3(256), 0, s,
                     (uint32_t*)p, n);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* ids, int64_t T, int k, int E, int64_t cap,
                           int tail_rows, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_slot, int32_t* slot_row, int32_t* n_kept,
                           int32_t* row_token, void* ws, hipStream_t s) {
  const int64_t Tk = T * (int64_t)k;
  const int nch = align_nchunks(Tk, E);
  if (Tk <= kSmallSlots) {
    const int ng = Tk <= kSmallSlots / 8 ? 1 : Tk <= kSmallSlots / 4 ? 2 : Tk <= kSmallSlots / 2 ? 4 : 8;
    const int nc = (int)MOE_CEIL_DIV(Tk, ng * 64);
    auto kern = ng == 1 ? k_align_small<1> : ng == 2 ? k_align_small<2>
              : ng == 4 ? k_align_small<4> : k_align_small<8>;
    hipLaunchKernelGGL(kern, dim3(1), dim3(1024), 0, s, ids, Tk, k, E, nc, cap, tail_rows,
                       counts, offsets, n_kept, sorted_slot, slot_row, row_token);
    return hipGetLastError();
  }
  int32_t* hist = (int32_t*)ws;
  const unsigned nblk = (unsigned)MOE_CEIL_DIV(nch, 4);
  if (nch > 0)
    hipLaunchKernelGGL(E <= 64 ? k_align_count<align_chunk_for(64)> : k_align_count<align_chunk_for(65)>,
                       dim3(nblk), dim3(256), 0, s, ids, Tk, E, nch, hist);
  hipLaunchKernelGGL(k_align_scan, dim3(1), dim3(256), 0, s, hist, E, nch, cap, tail_rows,
                     counts, offsets, n_kept);
  if (nch > 0)
    hipLaunchKernelGGL(E <= 64 ? k_align_scatter<align_chunk_for(64)> : k_align_scatter<align_chunk_for(65)>,
                       dim3(nblk), dim3(256), 0, s, ids, Tk, k, E, nch, cap,
                       hist, offsets, sorted_slot, slot_row, row_token);
  if (row_token && tail_rows > 0)
    hipLaunchKernelGGL(k_tail_tokens, dim3((unsigned)MOE_CEIL_DIV(tail_rows, 256)), dim3(256),
                       0, s, n_kept, tail_rows, row_token);
  return hipGetLastError();
}

size_t reroute_ws_bytes(int64_t T, int k, int E) {
  const int64_t Tk = T * (int64_t)k;
  const int nch = align_nchunks(Tk, E) > 0 ? align_nchunks(Tk, E) : 1;
  return align256((size_t)nch * E * sizeof(int32_t)) + align256((size_t)Tk * sizeof(int32_t) + 4) +
         align256((size_t)3 * E * sizeof(int32_t));
}

hipError_t launch_reroute(const int32_t* ids, const int32_t* backup, int nb, int64_t T, int k,
                          int E, int64_t cap, int tail_rows, const int32_t* counts,
                          int32_t* offsets, int32_t* sorted_slot, int32_t* slot_row,
                          int32_t* n_kept, int32_t* row_token, void* ws, hipStream_t s) {
  const int64_t Tk = T * (int64_t)k;
  if (Tk <= 0 || cap <= 0 || nb <= 0) return hipSuccess;
  const int nch = align_nchunks(Tk, E);
  char* p = (char*)ws;
  int32_t* hist2 = (int32_t*)p;  p += align256((size_t)nch * E * sizeof(int32_t));
  int32_t* props = (int32_t*)p;  p += align256((size_t)Tk * sizeof(int32_t) + 4);
  int32_t* meta = (int32_t*)p;
  hipLaunchKernelGGL(k_rr_props, dim3((unsigned)MOE_CEIL_DIV(T, 256)), dim3(256), 0, s, ids,
                     slot_row, backup, T, k, E, nb, props);
  const unsigned nblk = (unsigned)MOE_CEIL_DIV(nch, 4);
  hipLaunchKernelGGL(E <= 64 ? k_align_count<align_chunk_for(64)> : k_align_count<align_chunk_for(65)>,
                     dim3(nblk), dim3(256), 0, s, props, Tk, E, nch, hist2);
  hipLaunchKernelGGL(k_rr_scan, dim3(1), dim3(256), 0, s, hist2, E, nch, cap, tail_rows, counts,
                     offsets, n_kept, meta);
  hipLaunchKernelGGL(E <= 64 ? k_rr_place<align_chunk_for(64)> : k_rr_place<align_chunk_for(65)>,
                     dim3(nblk), dim3(256), 0, s, ids, props, Tk, k, E, nch, hist2,
                     offsets, meta, sorted_slot, slot_row, row_token);
  if (row_token && tail_rows > 0)
    hipLaunchKernelGGL(k_tail_tokens, dim3((unsigned)MOE_CEIL_DIV(tail_rows, 256)), dim3(256),
                       0, s, n_kept, tail_rows, row_token);
  return hipGetLastError();
}

hipError_t launch_gather(const void* X, const int32_t* sorted_slot, const int32_t* n_kept,
                         int64_t Tk, int k, int d, int elem_bytes, void* Xs, hipStream_t s) {
  if (Tk <= 0) return hipSuccess;
  const int vpr = d * elem_bytes / 16;
  hipLaunchKernelGGL(k_gather_rows, dim3((unsigned)Tk), dim3(256), 0, s, (const uint4*)X,
                     sorted_slot, n_kept, k, vpr, (uint4*)Xs);
  return hipGetLastError();
}

}  // namespace moe
